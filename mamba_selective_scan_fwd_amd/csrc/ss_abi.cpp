// ss_abi.cpp -- the C ABI of libss.so: host-side validation and dispatch.
// Every check runs before any HIP call; a failing check returns its status
// and leaves the device untouched.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstring>

#include "../../include/ss.h"
#include "ss_internal.h"

namespace {

constexpr int64_t kTile = 64;
constexpr int64_t kMaxDstate = 16;
constexpr int64_t kChPerBlock = 16;
// below this many wavefronts a forward splits the time axis into chunks
constexpr int64_t kTargetWaves = 1024;
// the largest grid, in workgroups of up to 512 threads, whose work-item count
// fits the 32-bit grid size of a dispatch
constexpr int64_t kMaxGrid = ((int64_t)1 << 23) - 1;
constexpr int64_t kMaxSeqlen = (int64_t)1 << 24;

bool aligned(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

int64_t elem_size(int32_t io) { return io == SS_F32 ? 4 : 2; }

ss_status check_problem(const ss_problem* p, bool need_seqlen) {
  if (!p) return SS_ERR_NULL_ARG;
  if (p->batch < 1 || p->dim < 1 || p->dstate < 1) return SS_ERR_BAD_SHAPE;
  if (need_seqlen && p->seqlen < 1) return SS_ERR_BAD_SHAPE;
  if (p->dstate > kMaxDstate) return SS_ERR_UNSUPPORTED;
  if (p->io_dtype != SS_F32 && p->io_dtype != SS_F16 && p->io_dtype != SS_BF16) return SS_ERR_BAD_DTYPE;
  // keep every element index far from int64 overflow and every grid within kMaxGrid
  const int64_t lim = (int64_t)1 << 40;
  if (p->batch > lim || p->dim > lim) return SS_ERR_BAD_SHAPE;
  // kernels address a row with 32-bit offsets
  if (need_seqlen && p->seqlen > kMaxSeqlen) return SS_ERR_BAD_SHAPE;
  const double ch = (double)p->batch * (double)p->dim;
  if (ch * (double)(need_seqlen ? p->seqlen : 1) * kMaxDstate > 9.0e18) return SS_ERR_BAD_SHAPE;
  if (ch / kChPerBlock * 2.0 > (double)kMaxGrid) return SS_ERR_BAD_SHAPE;
  return SS_OK;
}

struct FwdPlan {
  int64_t nchunks;
  int64_t chunk_len;
  size_t workspace;
};

// The forward's persistent work queue (problems that do not split time): units
// of kQueueChunk steps of a 16-channel block, for ragged rows or for more row
// blocks than the GPU holds at once.  Workspace: a control block, one flag per
// unit, one carried state per (channel, chunk).
// 2048 steps: a unit hands its state on through memory (a store, a flag and a
// load, each a trip to the memory side), which shorter units pay more often
// (units of 256, 512, 1024, 1536 and 2048 steps measured 0.63, 0.52, 0.47,
// 0.48 and 0.47 ms on the ragged mamba-2.8b workload; 0.71, 0.71, 0.69 and
// 0.69 ms from 512 up on the uniform layer).
constexpr int64_t kQueueChunk = 2048;
constexpr int64_t kQueueMaxRows = 256;
constexpr int64_t kFinalPerCu = 3;  // readout workgroups resident per CU (the headline's launch)
struct QueueLayout {
  int64_t chunks;
  size_t flags, carry, total;  // byte offsets and size
};
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
QueueLayout queue_layout(const ss_problem* p) {
  QueueLayout q;
  q.chunks = (p->seqlen + kQueueChunk - 1) / kQueueChunk;
  const int64_t ch_blocks = (p->dim + kChPerBlock - 1) / kChPerBlock;
  q.flags = 256;
  q.carry = q.flags + align256((size_t)(p->batch * ch_blocks * q.chunks) * 4);
  q.total = q.carry + (size_t)(p->batch * p->dim * q.chunks) * 16 * sizeof(float);
  return q;
}

// The time-chunked scan's workspace (one launch): a control block (its second
// word is the error word), then per (channel, chunk, state) the chunk pairs
// (P, S) and per (channel, group but the last, state) the group pairs, one
// 64-bit word each.  Groups hold G chunks, G the least power of two with
// G * G >= K, so that a chunk's entry state composes at most G - 1 chunk
// pairs and K / G group pairs.
struct ChunkLayout {
  int64_t group, ngroups;
  size_t pairs, gpairs, total;  // byte offsets and size
};
ChunkLayout chunk_layout(const ss_problem* p, int64_t nchunks) {
  ChunkLayout c;
  c.group = 1;
  while (c.group * c.group < nchunks) c.group *= 2;
  c.ngroups = (nchunks + c.group - 1) / c.group;
  c.pairs = 256;
  c.gpairs = c.pairs + (size_t)(p->batch * p->dim * nchunks) * 16 * sizeof(uint64_t);
  c.total = c.gpairs + (size_t)(p->batch * p->dim * (c.ngroups - 1)) * 16 * sizeof(uint64_t);
  return c;
}

FwdPlan plan_fwd(const ss_problem* p) {
  FwdPlan pl;
  const int64_t tiles = (p->seqlen + kTile - 1) / kTile;
  const int64_t ch_blocks = (p->dim + kChPerBlock - 1) / kChPerBlock;
  const int64_t waves = p->batch * ch_blocks * 4;
  int64_t k = 1;
  if (waves < kTargetWaves) {
    k = (kTargetWaves + waves - 1) / waves;  // at most kTargetWaves / 4 chunks
    if (k > tiles) k = tiles;
  }
  int64_t tiles_per_chunk = (tiles + k - 1) / k;
  // a time-chunked scan works on both halves of a chunk at once: an even
  // number of tiles per chunk
  if (k > 1) tiles_per_chunk += tiles_per_chunk & 1;
  pl.chunk_len = tiles_per_chunk * kTile;
  pl.nchunks = (p->seqlen + pl.chunk_len - 1) / pl.chunk_len;
  pl.workspace = pl.nchunks > 1 ? chunk_layout(p, pl.nchunks).total : 0;
  return pl;
}

ss_status from_hip(hipError_t e) { return e == hipSuccess ? SS_OK : SS_ERR_HIP; }

// A device buffer as a byte range; a null pointer or zero size is no buffer.
struct Span {
  const void* ptr;
  size_t n;
};
bool share_bytes(const Span& a, const Span& b) {
  if (!a.ptr || !b.ptr || !a.n || !b.n) return false;
  const uintptr_t x = (uintptr_t)a.ptr, y = (uintptr_t)b.ptr;
  return x < y + b.n && y < x + a.n;
}
// True when an output shares a byte with an input (unless it is that input
// itself and inplace[i][j] allows it) or with another output.
template <size_t NI, size_t NO>
bool conflict(const Span (&in)[NI], const Span (&out)[NO], const bool (*inplace)[NI] = nullptr) {
  for (size_t o = 0; o < NO; ++o) {
    for (size_t i = 0; i < NI; ++i)
      if (share_bytes(out[o], in[i]) &&
          !(inplace && inplace[o][i] && out[o].ptr == in[i].ptr && out[o].n == in[i].n))
        return true;
    for (size_t o2 = o + 1; o2 < NO; ++o2)
      if (share_bytes(out[o], out[o2])) return true;
  }
  return false;
}

}  // namespace

extern "C" {

const char* ss_status_str(ss_status s) {
  switch (s) {
    case SS_OK: return "ok";
    case SS_ERR_NULL_ARG: return "ss: a required pointer is NULL (or an optional input/output pair is half given)";
    case SS_ERR_BAD_SHAPE: return "ss: invalid problem size";
    case SS_ERR_BAD_DTYPE: return "ss: io_dtype must be SS_F32, SS_F16 or SS_BF16";
    case SS_ERR_MISALIGNED: return "ss: every tensor pointer must be 16-byte aligned";
    case SS_ERR_UNSUPPORTED:
      return "ss: unsupported request (a size outside the supported set, a workspace missing or too small, or "
             "overlapping buffers)";
    case SS_ERR_HIP: return "ss: HIP launch failed";
  }
  return "ss: unknown status";
}

size_t ss_ckpt_count(const ss_problem* p) {
  if (check_problem(p, true) != SS_OK) return 0;
  return (size_t)(p->batch * p->dim * ((p->seqlen + kTile - 1) / kTile) * p->dstate);
}

size_t ss_fwd_workspace_size(const ss_problem* p) {
  if (check_problem(p, true) != SS_OK) return 0;
  const FwdPlan pl = plan_fwd(p);
  if (pl.nchunks > 1 || p->batch > kQueueMaxRows) return pl.workspace;
  return queue_layout(p).total;
}

size_t ss_fwd_workspace_min(const ss_problem* p) {
  if (check_problem(p, true) != SS_OK) return 0;
  return plan_fwd(p).workspace;
}

ss_status ss_fwd(const ss_problem* p, const void* u, const void* delta, const float* A, const void* Bm,
                 const void* Cm, const float* D, const void* z, const float* delta_bias, const int32_t* lengths,
                 const int32_t* seq_idx, const float* h0, void* y, float* last_state, float* ckpt, void* workspace,
                 size_t workspace_bytes, void* stream) {
  return ss::fwd_checked(p, u, delta, A, Bm, Cm, D, z, delta_bias, lengths, seq_idx, h0, y, last_state, ckpt,
                         workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace ss {

size_t fwd_workspace_bytes(const ss_problem* p) { return ss_fwd_workspace_min(p); }
ss_status fwd_check_problem(const ss_problem* p) { return check_problem(p, true); }

ss_status fwd_checked(const ss_problem* p, const void* u, const void* delta, const float* A, const void* Bm,
                      const void* Cm, const float* D, const void* z, const float* delta_bias, const int32_t* lengths,
                      const int32_t* seq_idx, const float* h0, void* y, float* last_state, float* ckpt,
                      void* workspace, size_t workspace_bytes, void* stream) {
  ss_status s = check_problem(p, true);
  if (s != SS_OK) return s;
  if (!u || !delta || !A || !Bm || !Cm || !y) return SS_ERR_NULL_ARG;
  const void* ptrs[] = {u, delta, A, Bm, Cm, D, z, delta_bias, lengths, seq_idx, h0, y, last_state, ckpt, workspace};
  for (const void* q : ptrs)
    if (q && !aligned(q)) return SS_ERR_MISALIGNED;
  const FwdPlan pl = plan_fwd(p);
  if (pl.workspace > 0 && (!workspace || workspace_bytes < pl.workspace)) return SS_ERR_UNSUPPORTED;
  // the work queue: for ragged rows, or for more 16-channel row blocks than the
  // GPU holds at once when they do not fill its slots evenly; only with a
  // workspace that holds it (without one the same scan runs without the queue)
  bool queue = false;
  const QueueLayout ql = queue_layout(p);
  const int64_t ch_blocks = (p->dim + kChPerBlock - 1) / kChPerBlock;
  const int64_t slots = kFinalPerCu * ss::device_cus();
  if (pl.nchunks == 1 && p->batch <= kQueueMaxRows && workspace && workspace_bytes >= ql.total) {
    const int64_t G = p->batch * ch_blocks;
    queue = lengths != nullptr || (G > slots && G % slots != 0);
  }
  const size_t ws_used = queue ? ql.total : pl.workspace;
  {
    // y may be u, delta or z itself (each wave reads a tile's inputs before it writes the
    // tile's outputs); no other overlap between an output and any buffer
    const size_t io = (size_t)(p->batch * p->dim * p->seqlen) * elem_size(p->io_dtype);
    const size_t bc = (size_t)(p->batch * p->dstate * p->seqlen) * elem_size(p->io_dtype);
    const size_t st = (size_t)(p->batch * p->dim * p->dstate) * sizeof(float);
    const Span in[] = {{u, io}, {delta, io}, {z, io}, {Bm, bc}, {Cm, bc},
                       {A, (size_t)(p->dim * p->dstate) * sizeof(float)}, {D, (size_t)p->dim * sizeof(float)},
                       {delta_bias, (size_t)p->dim * sizeof(float)}, {lengths, (size_t)p->batch * 4},
                       {seq_idx, (size_t)(p->batch * p->seqlen) * 4}, {h0, st}};
    const Span out[] = {{y, io}, {last_state, st}, {ckpt, ss_ckpt_count(p) * sizeof(float)},
                        {ws_used ? workspace : nullptr, ws_used}};
    static const bool inplace[4][11] = {{true, true, true}};
    if (conflict(in, out, inplace)) return SS_ERR_UNSUPPORTED;
  }

  ss::FwdParams k{};
  k.io = p->io_dtype;
  k.softplus = p->delta_softplus != 0;
  k.u = u; k.delta = delta; k.z = z; k.Bm = Bm; k.Cm = Cm;
  k.A = A; k.D = D; k.bias = delta_bias; k.lengths = lengths; k.seq_idx = seq_idx; k.h0 = h0;
  k.y = y; k.last_state = last_state; k.ckpt = ckpt;
  k.batch = p->batch; k.dim = p->dim; k.dstate = p->dstate; k.seqlen = p->seqlen;
  k.chunk_len = pl.chunk_len;
  k.ch_blocks = (p->dim + kChPerBlock - 1) / kChPerBlock;
  k.ckpt_per_row = (p->seqlen + kTile - 1) / kTile;
  k.nchunks = (int32_t)pl.nchunks;
  if (pl.nchunks > 1) {
    const ChunkLayout cl = chunk_layout(p, pl.nchunks);
    char* ws = static_cast<char*>(workspace);
    k.q_ctrl = reinterpret_cast<int32_t*>(ws);
    k.pairs = reinterpret_cast<uint64_t*>(ws + cl.pairs);
    k.gpairs = reinterpret_cast<uint64_t*>(ws + cl.gpairs);
    k.nslots = (int64_t)((cl.total - cl.pairs) / sizeof(uint64_t));
    k.group = (int32_t)cl.group;
    k.ngroups = (int32_t)cl.ngroups;
  }
  if (queue) {
    char* ws = static_cast<char*>(workspace);
    k.q_ctrl = reinterpret_cast<int32_t*>(ws);
    k.q_flags = reinterpret_cast<int32_t*>(ws + ql.flags);
    k.q_carry = reinterpret_cast<float*>(ws + ql.carry);
    k.q_chunks = ql.chunks;
    k.chunk_len = kQueueChunk;
    k.nchunks = (int32_t)ql.chunks;
    const int64_t units = ql.chunks * p->batch * ch_blocks;
    k.q_grid = units < slots ? units : slots;
  }
  return from_hip(ss::launch_fwd(k, pl.nchunks, static_cast<hipStream_t>(stream)));
}

}  // namespace ss

extern "C" {

ss_status ss_fwd_step(const ss_problem* p, const void* u_t, const void* delta_t, const float* A, const void* B_t,
                      const void* C_t, const float* D, const void* z_t, const float* delta_bias,
                      const float* state_in, float* state_out, void* y_t, void* stream) {
  ss_status s = check_problem(p, false);
  if (s != SS_OK) return s;
  if (!u_t || !delta_t || !A || !B_t || !C_t || !state_in || !state_out || !y_t) return SS_ERR_NULL_ARG;
  const void* ptrs[] = {u_t, delta_t, A, B_t, C_t, D, z_t, delta_bias, state_in, state_out, y_t};
  for (const void* q : ptrs)
    if (q && !aligned(q)) return SS_ERR_MISALIGNED;
  // in-place is allowed; a partial overlap of the two state buffers is not
  const uintptr_t a0 = (uintptr_t)state_in, b0 = (uintptr_t)state_out;
  const uintptr_t bytes = (uintptr_t)(p->batch * p->dim * p->dstate) * sizeof(float);
  if (a0 != b0 && a0 < b0 + bytes && b0 < a0 + bytes) return SS_ERR_UNSUPPORTED;

  ss::StepParams k{};
  k.io = p->io_dtype;
  k.softplus = p->delta_softplus != 0;
  k.u = u_t; k.delta = delta_t; k.z = z_t; k.Bt = B_t; k.Ct = C_t;
  k.A = A; k.D = D; k.bias = delta_bias;
  k.state_in = state_in; k.state_out = state_out; k.y = y_t;
  k.batch = p->batch; k.dim = p->dim; k.dstate = p->dstate;
  return from_hip(ss::launch_step(k, static_cast<hipStream_t>(stream)));
}

namespace {
// The backward's own grids: a workgroup per (batch row, 64-step chunk,
// channel block) for the chunk aggregates, one per channel for the carry scan
// (which runs only when there is more than one chunk).
ss_status check_bwd(const ss_problem* p) {
  const ss_status s = check_problem(p, true);
  if (s != SS_OK) return s;
  const double chunks = (double)((p->seqlen + kTile - 1) / kTile);
  const double cblocks = (double)((p->dim + kChPerBlock - 1) / kChPerBlock);
  if ((double)p->batch * chunks * cblocks > (double)kMaxGrid) return SS_ERR_BAD_SHAPE;
  if (chunks > 1 && (double)p->batch * (double)p->dim > (double)kMaxGrid) return SS_ERR_BAD_SHAPE;
  return SS_OK;
}
}  // namespace

size_t ss_bwd_workspace_size(const ss_problem* p) {
  if (check_bwd(p) != SS_OK) return 0;
  const int64_t nchunks = (p->seqlen + kTile - 1) / kTile;
  return (size_t)3 * (size_t)(p->batch * p->dim * nchunks * 16) * sizeof(float);
}

ss_status ss_bwd(const ss_problem* p, const void* u, const void* delta, const float* A, const void* Bm,
                 const void* Cm, const float* D, const void* z, const float* delta_bias, const int32_t* seq_idx,
                 const float* ckpt, const void* dy, const float* dlast, void* du, void* ddelta, void* dz, float* dA,
                 float* dB, float* dC, float* dD, float* dbias, float* dh0, void* workspace, size_t workspace_bytes,
                 void* stream) {
  ss_status s = check_bwd(p);
  if (s != SS_OK) return s;
  if (!u || !delta || !A || !Bm || !Cm || !ckpt || !dy || !du || !ddelta || !dA || !dB || !dC)
    return SS_ERR_NULL_ARG;
  if ((z == nullptr) != (dz == nullptr) || (D == nullptr) != (dD == nullptr) ||
      (delta_bias == nullptr) != (dbias == nullptr))
    return SS_ERR_NULL_ARG;
  const void* ptrs[] = {u, delta, A, Bm, Cm, D, z, delta_bias, seq_idx, ckpt, dy, dlast, du, ddelta, dz, dA, dB, dC,
                        dD, dbias, dh0, workspace};
  for (const void* q : ptrs)
    if (q && !aligned(q)) return SS_ERR_MISALIGNED;
  const size_t need = ss_bwd_workspace_size(p);
  if (!workspace || workspace_bytes < need) return SS_ERR_UNSUPPORTED;
  {
    // no output (or the workspace) shares a byte with any other buffer
    const size_t io = (size_t)(p->batch * p->dim * p->seqlen) * elem_size(p->io_dtype);
    const size_t bc = (size_t)(p->batch * p->dstate * p->seqlen) * elem_size(p->io_dtype);
    const size_t bc32 = (size_t)(p->batch * p->dstate * p->seqlen) * sizeof(float);
    const size_t st = (size_t)(p->batch * p->dim * p->dstate) * sizeof(float);
    const size_t dn = (size_t)(p->dim * p->dstate) * sizeof(float), dv = (size_t)p->dim * sizeof(float);
    const Span in[] = {{u, io}, {delta, io}, {z, io}, {Bm, bc}, {Cm, bc}, {A, dn}, {D, dv}, {delta_bias, dv},
                       {seq_idx, (size_t)(p->batch * p->seqlen) * 4}, {ckpt, ss_ckpt_count(p) * sizeof(float)},
                       {dy, io}, {dlast, st}};
    const Span out[] = {{du, io}, {ddelta, io}, {dz, io}, {dA, dn}, {dB, bc32}, {dC, bc32},
                        {dD, dv}, {dbias, dv}, {dh0, st}, {workspace, need}};
    if (conflict(in, out)) return SS_ERR_UNSUPPORTED;
  }

  ss::BwdParams k{};
  k.io = p->io_dtype;
  k.softplus = p->delta_softplus != 0;
  k.u = u; k.delta = delta; k.z = z; k.Bm = Bm; k.Cm = Cm;
  k.A = A; k.D = D; k.bias = delta_bias; k.ckpt = ckpt; k.dy = dy;
  k.seq_idx = seq_idx; k.dlast = dlast; k.dh0 = dh0;
  k.du = du; k.ddelta = ddelta; k.dz = dz;
  k.dA = dA; k.dB = dB; k.dC = dC; k.dD = dD; k.dbias = dbias;
  k.batch = p->batch; k.dim = p->dim; k.dstate = p->dstate; k.seqlen = p->seqlen;
  k.ch_blocks = (p->dim + kChPerBlock - 1) / kChPerBlock;
  k.nchunks = (p->seqlen + kTile - 1) / kTile;
  const size_t per = (size_t)(p->batch * p->dim * k.nchunks * 16);
  float* ws = static_cast<float*>(workspace);
  k.gcarry = ws;
  k.aggP = ws + per;
  k.aggG = ws + 2 * per;
  return from_hip(ss::launch_bwd(k, static_cast<hipStream_t>(stream)));
}

namespace {
ss_status check_conv(const ss_conv_problem* p, bool need_seqlen) {
  if (!p) return SS_ERR_NULL_ARG;
  if (p->batch < 1 || p->dim < 1) return SS_ERR_BAD_SHAPE;
  if (need_seqlen && (p->seqlen < 1 || p->seqlen > kMaxSeqlen)) return SS_ERR_BAD_SHAPE;
  if (p->io_dtype != SS_F32 && p->io_dtype != SS_F16 && p->io_dtype != SS_BF16) return SS_ERR_BAD_DTYPE;
  if (p->width < 1 || p->width > 4 || p->reserved != 0) return SS_ERR_UNSUPPORTED;
  const int64_t lim = (int64_t)1 << 40;
  if (p->batch > lim || p->dim > lim) return SS_ERR_BAD_SHAPE;
  if (need_seqlen && (double)p->batch * (double)p->dim * (double)ss::conv_tblocks(p->seqlen) > (double)kMaxGrid)
    return SS_ERR_BAD_SHAPE;
  if (!need_seqlen && (double)p->batch * (double)p->dim / 256.0 > (double)kMaxGrid) return SS_ERR_BAD_SHAPE;
  return SS_OK;
}
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}
}  // namespace

ss_status ss_conv1d_fwd(const ss_conv_problem* p, const void* x, const float* w, const float* bias,
                        const int32_t* seq_idx, const float* conv_init, void* out, float* conv_final,
                        void* stream) {
  ss_status s = check_conv(p, true);
  if (s != SS_OK) return s;
  if (!x || !w || !out) return SS_ERR_NULL_ARG;
  const void* ptrs[] = {x, w, bias, seq_idx, conv_init, out, conv_final};
  for (const void* q : ptrs)
    if (q && !aligned(q)) return SS_ERR_MISALIGNED;
  const size_t bytes = (size_t)(p->batch * p->dim * p->seqlen * elem_size(p->io_dtype));
  {
    // no output shares a byte with an input or the other output (the window going out is
    // written by a row's last time block while its first reads the window coming in)
    const size_t win = (size_t)(p->batch * p->dim * (p->width - 1)) * sizeof(float);
    const Span in[] = {{x, bytes}, {w, (size_t)(p->dim * p->width) * sizeof(float)},
                       {bias, (size_t)p->dim * sizeof(float)}, {seq_idx, (size_t)(p->batch * p->seqlen) * 4},
                       {conv_init, win}};
    const Span outs[] = {{out, bytes}, {conv_final, win}};
    if (conflict(in, outs)) return SS_ERR_UNSUPPORTED;
  }
  ss::ConvParams k{};
  k.io = p->io_dtype; k.width = p->width; k.silu = p->silu != 0;
  k.x = x; k.w = w; k.bias = bias; k.seq_idx = seq_idx; k.conv_init = conv_init;
  k.out = out; k.conv_final = conv_final;
  k.batch = p->batch; k.dim = p->dim; k.seqlen = p->seqlen;
  k.tblocks = ss::conv_tblocks(p->seqlen);
  return from_hip(ss::launch_conv(k, static_cast<hipStream_t>(stream)));
}

ss_status ss_conv1d_step(const ss_conv_problem* p, const void* x_t, const float* w, const float* bias,
                         const float* window_in, float* window_out, void* out_t, void* stream) {
  ss_status s = check_conv(p, false);
  if (s != SS_OK) return s;
  if (!x_t || !w || !out_t || ((!window_in || !window_out) && p->width > 1)) return SS_ERR_NULL_ARG;
  const void* ptrs[] = {x_t, w, bias, window_in, window_out, out_t};
  for (const void* q : ptrs)
    if (q && !aligned(q)) return SS_ERR_MISALIGNED;
  const size_t wbytes = (size_t)(p->batch * p->dim * (p->width - 1)) * sizeof(float);
  if (window_in != window_out && wbytes && overlaps(window_in, wbytes, window_out, wbytes)) return SS_ERR_UNSUPPORTED;
  ss::ConvStepParams k{};
  k.io = p->io_dtype; k.width = p->width; k.silu = p->silu != 0;
  k.x = x_t; k.w = w; k.bias = bias; k.window_in = window_in; k.window_out = window_out; k.out = out_t;
  k.batch = p->batch; k.dim = p->dim;
  return from_hip(ss::launch_conv_step(k, static_cast<hipStream_t>(stream)));
}

namespace {
constexpr int64_t kSsdChunk = 256;
ss_status check_ssd(const ss_ssd_problem* p) {
  if (!p) return SS_ERR_NULL_ARG;
  if (p->batch < 1 || p->seqlen < 1 || p->nheads < 1 || p->ngroups < 1) return SS_ERR_BAD_SHAPE;
  if (p->io_dtype != SS_F16 && p->io_dtype != SS_BF16) return SS_ERR_BAD_DTYPE;
  if (p->headdim != 64) return SS_ERR_UNSUPPORTED;
  if (p->dstate != 32 && p->dstate != 64 && p->dstate != 96 && p->dstate != 128) return SS_ERR_UNSUPPORTED;
  if (p->nheads % p->ngroups != 0) return SS_ERR_UNSUPPORTED;
  // the kernels address a 256-step chunk of x or z (256 * nheads * 64 * 2
  // bytes) with 32-bit offsets; at most 2^30 bytes
  if (p->nheads > 32768) return SS_ERR_UNSUPPORTED;
  const int64_t lim = (int64_t)1 << 31;
  if (p->batch > lim || p->seqlen > lim || p->nheads > lim) return SS_ERR_BAD_SHAPE;
  const double nchunks = (double)((p->seqlen + kSsdChunk - 1) / kSsdChunk);
  if ((double)p->batch * nchunks * (double)p->nheads > (double)kMaxGrid) return SS_ERR_BAD_SHAPE;
  if ((double)p->batch * (double)p->nheads * (p->dstate / 32) > (double)kMaxGrid) return SS_ERR_BAD_SHAPE;
  if ((double)p->batch * (double)p->seqlen * (double)p->nheads * 64.0 > 9.0e18) return SS_ERR_BAD_SHAPE;
  return SS_OK;
}
size_t ssd_state_elems(const ss_ssd_problem* p) {
  const int64_t nchunks = (p->seqlen + kSsdChunk - 1) / kSsdChunk;
  return (size_t)(p->batch * nchunks * p->nheads) * (size_t)(64 * p->dstate);
}
}  // namespace

size_t ssd_cb_bytes(const ss_ssd_problem* p) {
  const int64_t nchunks = (p->seqlen + kSsdChunk - 1) / kSsdChunk;
  return (size_t)(p->batch * nchunks * p->ngroups) * (size_t)(kSsdChunk * kSsdChunk) * 2;
}

size_t ss_ssd_workspace_size(const ss_ssd_problem* p) {
  if (check_ssd(p) != SS_OK) return 0;
  return align256(ssd_state_elems(p) * 2) + align256(ssd_cb_bytes(p));
}

ss_status ss_ssd_fwd(const ss_ssd_problem* p, const void* x, const void* dt, const float* A, const void* Bm,
                     const void* Cm, const float* D, const void* z, const float* dt_bias, const int32_t* seq_idx,
                     const float* h0, void* y, float* final_state, void* workspace, size_t workspace_bytes,
                     void* stream) {
  ss_status s = check_ssd(p);
  if (s != SS_OK) return s;
  if (!x || !dt || !A || !Bm || !Cm || !y) return SS_ERR_NULL_ARG;
  // a row's document ids are read through one 32-bit range-checked view
  if (seq_idx && p->seqlen > ((int64_t)1 << 29)) return SS_ERR_UNSUPPORTED;
  const void* ptrs[] = {x, dt, A, Bm, Cm, D, z, dt_bias, seq_idx, h0, y, final_state, workspace};
  for (const void* q : ptrs)
    if (q && !aligned(q)) return SS_ERR_MISALIGNED;
  const size_t need = ss_ssd_workspace_size(p);
  if (!workspace || workspace_bytes < need) return SS_ERR_UNSUPPORTED;
  {
    // y may be x or z itself (a workgroup reads its own rows of x and z before it writes
    // them) and final_state may be h0 itself (each element is read and written by one
    // thread); no other overlap between an output or the workspace and an operand
    const size_t xb = (size_t)(p->batch * p->seqlen * p->nheads) * 64 * 2;
    const size_t dtb = (size_t)(p->batch * p->seqlen * p->nheads) * 2;
    const size_t bcb = (size_t)(p->batch * p->seqlen * p->ngroups * p->dstate) * 2;
    const size_t hb = (size_t)(p->batch * p->nheads) * 64 * (size_t)p->dstate * 4;
    const size_t vb = (size_t)p->nheads * 4;
    struct Span { const void* ptr; size_t n; };
    const Span in[] = {{x, xb},       {dt, dtb},      {A, vb},
                       {Bm, bcb},     {Cm, bcb},      {D, vb},
                       {z, xb},       {dt_bias, vb},  {seq_idx, (size_t)(p->batch * p->seqlen) * 4},
                       {h0, hb}};
    for (const Span& r : in) {
      if (!r.ptr) continue;
      if (overlaps(r.ptr, r.n, y, xb) && !(r.ptr == y && (r.ptr == x || r.ptr == z))) return SS_ERR_UNSUPPORTED;
      if (final_state && overlaps(r.ptr, r.n, final_state, hb) && !(r.ptr == final_state && r.ptr == h0))
        return SS_ERR_UNSUPPORTED;
      if (overlaps(r.ptr, r.n, workspace, need)) return SS_ERR_UNSUPPORTED;
    }
    if (final_state && overlaps(final_state, hb, y, xb)) return SS_ERR_UNSUPPORTED;
    if (overlaps(workspace, need, y, xb) || (final_state && overlaps(workspace, need, final_state, hb)))
      return SS_ERR_UNSUPPORTED;
  }
  const size_t e = ssd_state_elems(p);
  ss::SsdParams k{};
  k.io = p->io_dtype; k.softplus = p->dt_softplus != 0;
  k.x = x; k.dt = dt; k.A = A; k.Bm = Bm; k.Cm = Cm; k.D = D; k.z = z; k.dt_bias = dt_bias; k.h0 = h0;
  k.seq_idx = seq_idx;
  k.y = y; k.final_state = final_state;
  char* ws = static_cast<char*>(workspace);
  k.ws_entry = reinterpret_cast<uint16_t*>(ws);
  k.ws_cb = reinterpret_cast<uint16_t*>(ws + align256(e * 2));
  k.batch = p->batch; k.seqlen = p->seqlen; k.nheads = p->nheads; k.ngroups = p->ngroups; k.dstate = p->dstate;
  k.nchunks = (p->seqlen + kSsdChunk - 1) / kSsdChunk;
  return from_hip(ss::launch_ssd(k, static_cast<hipStream_t>(stream)));
}

ss_status ss_copy_probe(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return SS_ERR_NULL_ARG;
  if (!aligned(src) || !aligned(dst)) return SS_ERR_MISALIGNED;
  if (bytes % 16 != 0 || bytes == 0) return SS_ERR_BAD_SHAPE;
  return from_hip(ss::launch_copy(src, dst, (int64_t)bytes, static_cast<hipStream_t>(stream)));
}

ss_status ss_alu_probe(int32_t kind, int32_t workgroups, int32_t iters, int32_t lds_bytes, int64_t* out,
                       void* stream) {
  if (!out) return SS_ERR_NULL_ARG;
  if (!aligned(out)) return SS_ERR_MISALIGNED;
  if (kind < SS_PROBE_FMA || kind > SS_PROBE_SCAN_STEP) return SS_ERR_UNSUPPORTED;
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 20)) return SS_ERR_BAD_SHAPE;
  if (lds_bytes < 0 || lds_bytes > 65536) return SS_ERR_BAD_SHAPE;
  return from_hip(ss::launch_alu_probe(kind, workgroups, iters, lds_bytes, out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
