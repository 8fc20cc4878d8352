// ss_probe.hip -- measurement utilities (gfx950): a plain streaming copy for
// HBM bandwidth and traffic-counter calibration, and an issue-rate probe for
// the vector instructions the scan is made of.  Neither is part of the scan.
//
// The issue-rate probe times, on every wave, a fixed stream of one kind of
// instruction with the shader clock (s_memtime) and the constant 100 MHz
// clock (s_memrealtime), so that both the cost of an instruction in shader
// cycles and the clock the chip actually ran at are measured.  Kinds:
//   FMA        v_fma_f32, 16 independent chains
//   EXP        v_exp_f32, 16 independent chains
//   DPP_MUL    v_mul_f32 with a DPP row broadcast of its first operand (how the
//              scan hands Delta and Delta*u to the lanes of a channel)
//   SCAN_STEP  the scan's per-lane step, 16 steps per iteration:
//              a = exp2(bcast(Delta) * A log2e); h = a h + bcast(Delta u) B
//              (two DPP-folded multiplies, one exp, one FMA; one h chain)
// Each iteration holds 16 instructions of the kind (16 steps of 4 for
// SCAN_STEP).  Values never leave registers; a store that the data can never
// trigger keeps the chains alive.  Every wave also records where it ran (XCD,
// shader engine, CU, SIMD), so that rates are taken per SIMD over the waves
// it actually held: the dispatcher need not spread workgroups evenly over
// the CUs.  An optional block of unused LDS per workgroup limits how many
// workgroups share a CU, as a kernel's own LDS use does.
#include <utility>

#include "ss_device.h"
#include "ss_internal.h"

namespace ss {

namespace {

// Plain device copy, 16 bytes per lane per iteration: the reference kernel
// for HBM bandwidth and for calibrating traffic counters.
__global__ void __launch_bounds__(256) ss_copy_kernel(const float4* __restrict__ src, float4* __restrict__ dst,
                                                      int64_t n16) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n16; i += stride) dst[i] = src[i];
}

template <int... J>
__device__ __forceinline__ void dpp_mul_chains(float (&acc)[16], float src, std::integer_sequence<int, J...>) {
  ((acc[J] = row_bcast<J>(src) * acc[J]), ...);
}

template <int... J>
__device__ __forceinline__ void scan_steps(float& h, float dt, float dtu, float A2, const float (&b)[16],
                                           std::integer_sequence<int, J...>) {
  ((h = fmaf(exp2_hw(row_bcast<J>(dt) * A2), h, row_bcast<J>(dtu) * b[J])), ...);
}

// Where this wave runs: the hardware's wave id register (SIMD, CU, shader
// engine) and the XCD, so that the host can count the waves each SIMD held.
__device__ __forceinline__ int64_t wave_place() {
  uint32_t hw, xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  return ((int64_t)xcc << 32) | (int64_t)hw;
}

template <int KIND>
__global__ void __launch_bounds__(256) ss_alu_probe_kernel(int32_t iters, float seed, int64_t* __restrict__ out) {
  const int lane = threadIdx.x % 64;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / 64;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = seed + 0.001f * (float)(i + lane);
  float src = seed * 0.5f + 0.01f * (float)lane;
  // FMA operands in registers (an inline literal would lengthen the encoding)
  const float fa = fresh(seed * 1.998f), fb = fresh(seed * 0.002f);
  float h = 0.0f;
  const float A2 = -0.3f * (float)(lane % 16 + 1) * kLog2e;
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  __builtin_amdgcn_sched_barrier(0);
#pragma nounroll
  for (int it = 0; it < iters; ++it) {
    if constexpr (KIND == SS_PROBE_FMA) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = fmaf(acc[i], fa, fb);
    } else if constexpr (KIND == SS_PROBE_EXP) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = exp2_hw(-acc[i]);
    } else if constexpr (KIND == SS_PROBE_DPP_MUL) {
      // a fresh source each iteration, so the broadcasts cannot be hoisted
      src = fresh(src);
      dpp_mul_chains(acc, src, std::make_integer_sequence<int, 16>{});
    } else {
      // the scan's step: Delta and Delta*u of 16 steps owned one per lane
      const float dt = fresh(src);
      const float dtu = fresh(acc[0]);
      scan_steps(h, dt, dtu, A2, acc, std::make_integer_sequence<int, 16>{});
      h = fresh(h);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float sum = h;
#pragma unroll
  for (int i = 0; i < 16; ++i) sum += acc[i];
  const int64_t place = wave_place();
  if (lane == 0) {
    out[wave * 6 + 0] = (int64_t)c0;
    out[wave * 6 + 1] = (int64_t)c1;
    out[wave * 6 + 2] = (int64_t)r0;
    out[wave * 6 + 3] = (int64_t)r1;
    out[wave * 6 + 4] = place;
    out[wave * 6 + 5] = 0;
  }
  // never true for the data above (sum is finite); keeps every chain live
  if (sum == -1234.5f) out[wave * 6 + 0] = -1;
}

template <int KIND>
hipError_t launch_probe_kind(int32_t workgroups, int32_t iters, int32_t lds_bytes, int64_t* out, hipStream_t st) {
  hipLaunchKernelGGL((ss_alu_probe_kernel<KIND>), dim3((uint32_t)workgroups), dim3(256), (uint32_t)lds_bytes, st,
                     iters, 0.5f, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(ss_copy_kernel, dim3((uint32_t)blocks), dim3(256), 0, st,
                     reinterpret_cast<const float4*>(src), reinterpret_cast<float4*>(dst), n16);
  return hipGetLastError();
}

hipError_t launch_alu_probe(int32_t kind, int32_t workgroups, int32_t iters, int32_t lds_bytes, int64_t* out,
                            hipStream_t st) {
  switch (kind) {
    case SS_PROBE_FMA: return launch_probe_kind<SS_PROBE_FMA>(workgroups, iters, lds_bytes, out, st);
    case SS_PROBE_EXP: return launch_probe_kind<SS_PROBE_EXP>(workgroups, iters, lds_bytes, out, st);
    case SS_PROBE_DPP_MUL: return launch_probe_kind<SS_PROBE_DPP_MUL>(workgroups, iters, lds_bytes, out, st);
    default: return launch_probe_kind<SS_PROBE_SCAN_STEP>(workgroups, iters, lds_bytes, out, st);
  }
}

}  // namespace ss
