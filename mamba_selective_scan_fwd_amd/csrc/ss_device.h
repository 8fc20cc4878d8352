// ss_device.h -- device helpers shared by the selective-scan kernels (gfx950).
// Internal to libss.so; not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ss.h"

namespace ss {

constexpr int kTile = 64;      // time steps per tile; also the checkpoint interval
constexpr int kStates = 16;    // state lanes per channel (dstate is padded to 16)
constexpr int kChPerWave = 4;  // 64-lane wavefront = 4 channels x 16 states
constexpr int kWaves = 4;      // waves per workgroup
constexpr int kChPerBlock = kChPerWave * kWaves;  // 16 channels per workgroup
constexpr int kThreads = 64 * kWaves;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- I/O element conversions (data tensors are fp32, fp16 or bf16) --------
template <int IO> struct io_elem;
template <> struct io_elem<SS_F32> { using T = float; };
template <> struct io_elem<SS_F16> { using T = _Float16; };
template <> struct io_elem<SS_BF16> { using T = uint16_t; };

template <int IO> __device__ __forceinline__ float to_f32(typename io_elem<IO>::T v);
template <> __device__ __forceinline__ float to_f32<SS_F32>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<SS_F16>(_Float16 v) { return (float)v; }
template <> __device__ __forceinline__ float to_f32<SS_BF16>(uint16_t v) {
  return __uint_as_float((uint32_t)v << 16);
}

template <int IO> __device__ __forceinline__ typename io_elem<IO>::T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<SS_F32>(float v) { return v; }
template <> __device__ __forceinline__ _Float16 from_f32<SS_F16>(float v) { return (_Float16)v; }
template <> __device__ __forceinline__ uint16_t from_f32<SS_BF16>(float v) {
  // round to nearest even in hardware (v_cvt_pk_bf16_f32 on gfx950)
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// ---- buffer-resource access (hardware range check: loads past num_records
// return 0, stores past it are dropped).  The base must be wave-uniform.
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
constexpr uint32_t kOffNone = 0x7fffffffu;  // an offset that is always out of range

// raw element bits, kept in their storage width until converted at the point
// of use (so a load's wait is not forced early by a widening instruction)
template <int IO> struct raw_elem { using T = uint16_t; };
template <> struct raw_elem<SS_F32> { using T = uint32_t; };
template <int IO> using raw_t = typename raw_elem<IO>::T;

template <int IO>
__device__ __forceinline__ raw_t<IO> bload(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  if constexpr (IO == SS_F32)
    return __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0);
  else
    return __builtin_amdgcn_raw_buffer_load_b16(r, byte_off, 0, 0);
}
template <int IO>
__device__ __forceinline__ float bits_f32(raw_t<IO> v) {
  if constexpr (IO == SS_F32)
    return __uint_as_float(v);
  else if constexpr (IO == SS_F16)
    return (float)__builtin_bit_cast(_Float16, v);
  else
    return __uint_as_float((uint32_t)v << 16);
}
template <int IO>
__device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float v) {
  if constexpr (IO == SS_F32)
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, byte_off, 0, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, from_f32<IO>(v)), r, byte_off, 0, 0);
}
template <int IO> constexpr uint32_t io_bytes() { return IO == SS_F32 ? 4u : 2u; }

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ---- packed documents ("niverel-mamba" README, "seq_idx strict reset") -----
// Lane i of a wave holds the document ids of step t = t0 + i and of t - 1
// (raw 32-bit words from a range-checked view of the row's ids; t - 1 = -1
// reads as out of range).  Bit i of the result is set when step t starts a new
// document inside [1, t_end): the state is zero before that step.
__device__ __forceinline__ uint64_t doc_starts(uint32_t id_t, uint32_t id_prev, int t, int t_end) {
  return __builtin_amdgcn_ballot_w64(t > 0 && t < t_end && id_t != id_prev);
}
__device__ __forceinline__ void load_doc_ids(__amdgpu_buffer_rsrc_t ids, int t, uint32_t& id_t, uint32_t& id_prev) {
  id_t = __builtin_amdgcn_raw_buffer_load_b32(ids, (uint32_t)t * 4u, 0, 0);
  id_prev = __builtin_amdgcn_raw_buffer_load_b32(ids, (uint32_t)(t - 1) * 4u, 0, 0);
}
// decay of step S of a tile with the reset applied: a new document multiplies
// the carried state by zero
template <bool RESET, int S>
__device__ __forceinline__ float reset_decay(float a, uint64_t starts) {
  if constexpr (RESET) return ((starts >> S) & 1ull) ? 0.0f : a;
  else return a;
}

template <int IO>
__device__ __forceinline__ float load_io(const void* base, int64_t i) {
  return to_f32<IO>(reinterpret_cast<const typename io_elem<IO>::T*>(base)[i]);
}
template <int IO>
__device__ __forceinline__ void store_io(void* base, int64_t i, float v) {
  reinterpret_cast<typename io_elem<IO>::T*>(base)[i] = from_f32<IO>(v);
}

// ---- fast transcendental pieces (hardware exp2/log2/rcp) -------------------
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^-|x|).  For e in (0, 1],
// w = fl(1 + e) carries a rounding error eps = (w - 1) - e, which is exact to
// evaluate (w - 1 is exact by Sterbenz).  log1p(e) = log(w) - eps / w +
// O(eps^2), and eps / w = eps to within e * eps, so
//   log1p(e) = ln2 * log2(w) + (e - (w - 1))
// to a few ulp relative, for every e (when w rounds to 1 the result is e
// itself).  max(x, 0) = (x + |x|) / 2 exactly.  Two transcendentals, no
// division, no clamp.
__device__ __forceinline__ float softplus_f(float x) {
  const float e = exp2_hw(-fabsf(x) * kLog2e);
  const float w = 1.0f + e;
  const float d = e - (w - 1.0f);
  return fmaf(0.5f, x + fabsf(x), fmaf(kLn2, log2_hw(w), d));
}

// d softplus / dx = sigmoid(x)
__device__ __forceinline__ float sigmoid_f(float x) { return rcp_hw(1.0f + exp2_hw(-x * kLog2e)); }

// SiLU(z) = z * sigmoid(z)
__device__ __forceinline__ float silu_f(float z) { return z * sigmoid_f(z); }

// An opaque copy of v.  Values derived from it are not merged with values
// derived from v earlier, and, being ordered with scheduling barriers, it pins
// the computation of v before the barrier that follows it: without such pins
// the compiler floats the arithmetic of every unrolled block past the
// barriers and keeps all blocks' broadcasts and exponentials live at once.
__device__ __forceinline__ float fresh(float v) {
  asm volatile("" : "+v"(v));
  return v;
}
// The same for a per-lane integer: addresses computed from it are rebuilt
// where they are used instead of being kept live (or spilled) from an
// earlier computation.
template <typename T>
__device__ __forceinline__ T opaque(T v) {
  asm volatile("" : "+v"(v));
  return v;
}

// ---- cross-lane moves inside a 16-lane DPP row ------------------------------
// value of lane J of this lane's row (DPP row_newbcast; folds into the VALU
// instruction that consumes it)
template <int J>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + J, 0xf, 0xf, true));
}
// value of lane (l + K) mod 16 of this lane's row (DPP row_ror)
template <int K>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + K, 0xf, 0xf, false));
}
// value of lane l - K of this lane's row, 0 for the first K lanes (DPP row_shr
// with bound_ctrl)
template <int K>
__device__ __forceinline__ float row_shr(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + K, 0xf, 0xf, true));
}
// inclusive running sum over the lanes 0..l of this lane's row
__device__ __forceinline__ float row_scan(float v) {
  v += row_shr<1>(v);
  v += row_shr<2>(v);
  v += row_shr<4>(v);
  v += row_shr<8>(v);
  return v;
}
// sum over the 16 lanes of a row, result in every lane of the row
__device__ __forceinline__ float row_sum(float v) {
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  v += row_ror<1>(v);
  return v;
}

// The SIMD's issue arbiter serves the oldest of equally ranked waves first, so
// of the waves that share a SIMD the first to arrive races ahead and the last
// one finishes alone, with the SIMD idle between its instructions.  A wave
// that walks a sequence therefore lowers its own rank as its work proceeds:
// 3 in the first half, 2 to three quarters, 1 to seven eighths, 0 after.
// Whenever a wave passes a mark the waves behind it are served first until
// they pass it too, so they all reach the last eighth close together and only
// that stretch is served oldest first.
__device__ __forceinline__ void rank_by_progress(int done, int total) {
  const int e = total > 0 ? (int)(((int64_t)done * 8) / total) : 0;
  if (e < 4) __builtin_amdgcn_s_setprio(3);
  else if (e < 6) __builtin_amdgcn_s_setprio(2);
  else if (e < 7) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Workgroup index remapped so that consecutive logical blocks share an XCD
// (MI355X dispatches workgroups round-robin over its 8 XCDs, each with its
// own L2): logical blocks that read the same B/C rows then hit one L2.
__device__ __forceinline__ uint32_t xcd_logical_block() {
  const uint32_t nb = gridDim.x, bid = blockIdx.x;
  const uint32_t per = nb / 8u, rem = nb % 8u;
  const uint32_t xcd = bid % 8u, local = bid / 8u;
  return xcd < rem ? xcd * (per + 1u) + local : rem * (per + 1u) + (xcd - rem) * per + local;
}

}  // namespace ss
