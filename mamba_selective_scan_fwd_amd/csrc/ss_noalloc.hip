// ss_noalloc.hip -- ss_fwd_noalloc: the forward scan for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  It is ss_fwd with its workspace (the
// time-chunked scan's chunk and group pairs, or the work queue of a ragged
// problem when it fits) taken from a fixed array in device memory instead of
// from the caller.
//
// The array lives for the life of the process, one copy per GPU that the
// library runs on.  Every call on a GPU uses that GPU's copy: calls that
// overlap in time on one GPU (on different streams) race on it.  Nothing in
// it needs clearing by the caller: a kernel at the start of every call that
// uses it clears what that call polls (the time-chunked scan's pair slots and
// counter, the queue's counter and flags).
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/ss.h"
#include "ss_internal.h"

namespace {

// Largest forward workspace any valid problem needs: the scan splits time only
// while the problem has fewer than 1024 wavefronts (4 per 16 channels), into
// at most ceil(1024 / waves) chunks, so batch * dim * chunks <= 8188 and the
// 64-bit pair slots of every (channel, chunk or group, state) take at most
// 1.05 MB.
constexpr size_t kScratchBytes = (size_t)2 << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of this GPU's copy of `scratch`, looked up once per
// device with that device current (in host code the array's name is only a
// stand-in for it).  Null when the runtime cannot give it.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

size_t ss_fwd_noalloc_max_workspace(void) { return kScratchBytes; }

ss_status ss_fwd_noalloc(const ss_problem* p, const void* u, const void* delta, const float* A, const void* Bm,
                         const void* Cm, const float* D, const void* z, const float* delta_bias,
                         const int32_t* lengths, const int32_t* seq_idx, const float* h0, void* y,
                         float* last_state, float* ckpt, void* stream) {
  const ss_status bad = ss::fwd_check_problem(p);
  if (bad != SS_OK) return bad;
  if (ss::fwd_workspace_bytes(p) > kScratchBytes) return SS_ERR_UNSUPPORTED;  // the least the scan needs
  // the whole array is offered: a problem whose optional work queue fits it
  // uses the queue, others run without it (same results)
  void* ws = scratch_ptr();
  if (!ws) return SS_ERR_HIP;
  return ss::fwd_checked(p, u, delta, A, Bm, Cm, D, z, delta_bias, lengths, seq_idx, h0, y, last_state, ckpt,
                         ws, kScratchBytes, stream);
}

}  // extern "C"
