// C ABI of the retention library: argument validation, planning and launches.
//
// Validation runs entirely on the host and before any HIP call, so invalid or
// unsupported arguments are reported without touching a device. Planning is a
// pure function of the sizes: it picks the MFMA kernels for bf16 shapes they
// cover and the generic vector-ALU kernels otherwise, and it sizes the
// chunkwise workspace.
#include <algorithm>
#include <cfloat>
#include <climits>
#include <cmath>
#include <cstdint>

#include "kernels.h"
#include "retention.h"

namespace {

using ret::Dims;
using ret::GnArgs;
using ret::HeadDecay;

static_assert(ret::kScratchBytes == RETENTION_NOALLOC_MAX_WORKSPACE_BYTES, "scratch size");

constexpr size_t kAlign = 256;
constexpr int kMfmaRows = 64;            // MFMA kernels need chunk % 64 == 0
constexpr int64_t kWalkTargetBlocks = 512;  // segment the walk below this many workgroups
// The single-pass kernel runs one workgroup per (head, 256-column v tile);
// below this many of them the two-stage path, which parallelises over query
// blocks, keeps more of the GPU busy.
constexpr int64_t kFusedMinUnits = 192;
// Above this chunk length the single pass re-reads each chunk's keys and
// values once per 64-row query block (its state takes the registers a
// longer block would need) and measures slower than the two stages.
constexpr int kFusedMaxChunk = 128;
// With fewer (head, v tile) pairs than kFusedMinUnits the sequences are cut
// into segments (walked in parallel from states a first pass computes) until
// there are about kFusedTargetUnits units, one per CU, keeping at least
// kFusedMinChunksPerSeg chunks per segment.
constexpr int64_t kFusedTargetUnits = 256;
constexpr int kFusedMinChunksPerSeg = 4;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool valid_dtype(int dtype) { return dtype == RET_F32 || dtype == RET_BF16; }

int check_sizes(int B, int H, int N, int dk, int dv, int dtype) {
  if (B <= 0 || H <= 0 || N <= 0 || dk <= 0 || dv <= 0) return RET_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return RET_ERR_INVALID_ARG;
  if (H > RETENTION_MAX_HEADS || dk > RETENTION_MAX_DK || dv > RETENTION_MAX_DV) return RET_ERR_UNSUPPORTED;
  // Grid sizes: the generic output kernel launches one block per (b, h, n).
  if (static_cast<int64_t>(B) * H * N >= (int64_t{1} << 31)) return RET_ERR_UNSUPPORTED;
  return RET_OK;
}

int check_gamma(const float* gamma_host, int H, HeadDecay* decay) {
  if (!gamma_host) return RET_ERR_INVALID_ARG;
  for (int h = 0; h < H; ++h) {
    const float g = gamma_host[h];
    if (!std::isfinite(g) || !(g > 0.0f) || !(g < 1.0f)) return RET_ERR_INVALID_ARG;
  }
  if (decay) {
    for (int h = 0; h < RETENTION_MAX_HEADS; ++h)
      decay->log2g[h] = h < H ? static_cast<float>(std::log2(static_cast<double>(gamma_host[h]))) : 0.0f;
  }
  return RET_OK;
}

int check_gn(const retention_gn_t* gn, GnArgs* out) {
  out->enabled = 0;
  out->eps = 0.0f;
  out->weight = nullptr;
  out->bias = nullptr;
  out->gate = nullptr;
  if (!gn) return RET_OK;
  if (!std::isfinite(gn->eps) || gn->eps < 0.0f) return RET_ERR_INVALID_ARG;
  out->enabled = 1;
  out->eps = gn->eps;
  out->weight = gn->weight;
  out->bias = gn->bias;
  out->gate = gn->gate;
  return RET_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? RET_OK : RET_ERR_HIP; }

// Whether [a, a + an) and [b, b + bn) share a byte.
bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bn && y < x + an;
}

// Whether O ([B, H, N, dv]) shares bytes with Q, K ([B, H, N, dk]) or V, or a
// gate (laid out like O, may be null) with O: the kernels write O while other
// workgroups still read the inputs (and the gate at the positions they store).
bool output_overlaps(const void* q, const void* k, const void* v, const void* o, const void* gate, int B, int H,
                     int N, int dk, int dv, int dtype) {
  const size_t es = dtype == RET_F32 ? 4 : 2;
  const size_t tok = static_cast<size_t>(B) * H * N;
  const size_t nk = tok * dk * es, nv = tok * dv * es;
  return overlaps(o, nv, q, nk) || overlaps(o, nv, k, nk) || overlaps(o, nv, v, nv) ||
         (gate && overlaps(gate, nv, o, nv));
}

// A chunk at least as long as the sequence is one chunk: every such length
// gives the same result. It is brought down to the sequence length rounded up
// to a multiple of the MFMA block height (so the MFMA kernels stay eligible),
// which keeps every later product of a chunk index and the chunk length
// within int range.
int effective_chunk(int N, int chunk) {
  if (chunk <= N) return chunk;
  const int64_t up = (static_cast<int64_t>(N) + kMfmaRows - 1) / kMfmaRows * kMfmaRows;
  return static_cast<int>(std::min<int64_t>(chunk, up <= INT_MAX ? up : N));
}

// Chunkwise execution plan: the single-pass kernel (fused), or the two stages
// (state walk, then output) on the MFMA or the generic kernels.
struct ChunkPlan {
  bool fused;
  bool mfma;
  int nchunks;
  int chunks_per_seg;
  int nseg;
  size_t states_bytes;  // per-chunk states (two stages); the mailbox (single pass)
  size_t seg_bytes;     // segment end states (nseg > 1)
  size_t in_bytes;      // single pass with segments: a copy of state_in when state_out aliases it
  size_t total;
};

// Segments of the single pass for these sizes: 1 when the heads alone give
// enough units, 0 when neither they nor segments of at least
// kFusedMinChunksPerSeg chunks do (then the two stages run).
int fused_segments(int B, int H, int dk, int dv, int chunk, int dtype, int nchunks) {
  if (dtype != RET_BF16 || chunk > kFusedMaxChunk || !ret::fused_supports(dk, dv, chunk)) return 0;
  const int64_t base = static_cast<int64_t>(B) * H * (dv / 256);
  if (base >= kFusedMinUnits) return 1;
  int64_t nseg = (kFusedTargetUnits + base - 1) / base;
  nseg = std::min<int64_t>(nseg, nchunks / kFusedMinChunksPerSeg);
  if (nseg < 2 || base * nseg < kFusedMinUnits) return 0;
  return static_cast<int>(nseg);
}

// `stages`: plan the two stages even where the single-pass kernel applies
// (the explicit stage entry points).
ChunkPlan plan_chunkwise(int B, int H, int N, int dk, int dv, int chunk, int dtype, bool stages = false) {
  ChunkPlan p{};
  p.nchunks = static_cast<int>((static_cast<int64_t>(N) + chunk - 1) / chunk);
  const int fseg = stages ? 0 : fused_segments(B, H, dk, dv, chunk, dtype, p.nchunks);
  if (fseg > 0) {
    p.fused = true;
    p.chunks_per_seg = (p.nchunks + fseg - 1) / fseg;
    p.nseg = (p.nchunks + p.chunks_per_seg - 1) / p.chunks_per_seg;
    const size_t heads = static_cast<size_t>(B) * H;
    const size_t dkdv = static_cast<size_t>(dk) * dv;
    p.states_bytes = align_up(ret::fused_workspace_bytes(static_cast<int64_t>(heads) * p.nseg, dv));
    p.seg_bytes = p.nseg > 1 ? align_up(heads * p.nseg * dkdv * sizeof(float)) : 0;
    p.in_bytes = p.nseg > 1 ? align_up(heads * dkdv * sizeof(float)) : 0;
    p.total = p.states_bytes + p.seg_bytes + p.in_bytes;
    return p;
  }
  p.mfma = dtype == RET_BF16 && ret::mfma_supports(dk, dv) && chunk % kMfmaRows == 0;
  p.nchunks = static_cast<int>((static_cast<int64_t>(N) + chunk - 1) / chunk);
  const size_t heads = static_cast<size_t>(B) * H;
  const size_t dkdv = static_cast<size_t>(dk) * dv;
  if (p.mfma) {
    const int64_t per_seg = static_cast<int64_t>(heads) * ret::walk_tiles_per_head(heads, dk, dv);
    int64_t want = ret::walk_wide(heads, dk, dv) ? 1 : (kWalkTargetBlocks + per_seg - 1) / per_seg;
    if (want < 1) want = 1;
    if (want > p.nchunks) want = p.nchunks;
    p.chunks_per_seg = static_cast<int>((p.nchunks + want - 1) / want);
    p.nseg = (p.nchunks + p.chunks_per_seg - 1) / p.chunks_per_seg;
    p.states_bytes = align_up(heads * p.nchunks * dkdv * sizeof(uint16_t));
    p.seg_bytes = p.nseg > 1 ? align_up(heads * p.nseg * dkdv * sizeof(float)) : 0;
  } else {
    p.chunks_per_seg = p.nchunks;
    p.nseg = 1;
    p.states_bytes = align_up(heads * p.nchunks * dkdv * sizeof(float));
    p.seg_bytes = 0;
  }
  p.total = p.states_bytes + p.seg_bytes;
  return p;
}

// Shared validation of the chunkwise entry points (no HIP calls).
int check_chunkwise(const float* gamma_host, int B, int H, int N, int dk, int dv, int* chunk, int dtype,
                    const retention_gn_t* gn, const void* workspace, size_t workspace_bytes, GnArgs* g,
                    ChunkPlan* plan, HeadDecay* decay, bool stages = false) {
  if (*chunk <= 0) return RET_ERR_INVALID_ARG;
  int st = check_sizes(B, H, N, dk, dv, dtype);
  if (st != RET_OK) return st;
  *chunk = effective_chunk(N, *chunk);
  st = check_gamma(gamma_host, H, nullptr);
  if (st != RET_OK) return st;
  st = check_gn(gn, g);
  if (st != RET_OK) return st;
  *plan = plan_chunkwise(B, H, N, dk, dv, *chunk, dtype, stages);
  if (plan->total > 0 && (!workspace || workspace_bytes < plan->total)) return RET_ERR_INVALID_ARG;
  check_gamma(gamma_host, H, decay);
  return RET_OK;
}

hipError_t launch_states(const ChunkPlan& p, const void* k, const void* v, const float* state_in, float* state_out,
                         char* ws, const Dims& d, int chunk, int dtype, const HeadDecay& decay, hipStream_t s) {
  if (p.mfma) {
    uint16_t* states = reinterpret_cast<uint16_t*>(ws);
    float* segs = p.seg_bytes ? reinterpret_cast<float*>(ws + p.states_bytes) : nullptr;
    return ret::launch_mfma_state_walk(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), state_in,
                                       state_out, states, segs, p.chunks_per_seg, d, chunk, decay, s);
  }
  return ret::launch_generic_state_walk(dtype, k, v, state_in, state_out, reinterpret_cast<float*>(ws), d, chunk,
                                        decay, s);
}

hipError_t launch_output(const ChunkPlan& p, const void* q, const void* k, const void* v, void* o, const char* ws,
                         bool state0, const Dims& d, int chunk, int dtype, const HeadDecay& decay, const GnArgs& g,
                         hipStream_t s, bool accumulate = false) {
  if (p.mfma) {
    return ret::launch_mfma_chunk_out(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                      static_cast<const uint16_t*>(v), reinterpret_cast<const uint16_t*>(ws), state0,
                                      static_cast<uint16_t*>(o), d, chunk, decay, g, accumulate, s);
  }
  return ret::launch_generic_chunk_out(dtype, q, k, v, reinterpret_cast<const float*>(ws), state0, o, d, chunk,
                                       decay, g, accumulate, s);
}

// Backward plan: operand copies, partial results, state transforms and the
// workspace of the chunkwise calls, laid out one after another.
constexpr int kPartWidth = 256;  // widest query/key dimension the MFMA kernels take

struct BackwardPlan {
  // Single-pass plan: every retention on the single-pass kernel, reading the
  // operands in place (row pitches, reverse order), one launch per 256-wide
  // part for the dQ and dK retentions together; no copies.
  bool direct;
  size_t mail;  // direct: exchange words of the widest launch
  int nparts;  // parts of the dv-wide query/key dimension of the dQ and dK retentions
  int part_w;
  size_t qf, kf, dof, oa, dos, vs, dofs, vfs, kpart;  // byte offsets (token-row buffers)
  size_t s_a, s_t, s_0t, s_nt;                               // fp32 state buffers
  size_t cw;                                                 // chunkwise workspace
  size_t cw_bytes;
  size_t total;
};

// Whether the backward runs directly on the single-pass kernel: bf16, the
// retentions' widths and chunk within its range, enough units for each launch
// without segments ((head, v tile) for dV; (retention, head, v tile) for a
// part of dQ and dK together), and reverse-order offsets within 2^30 bytes.
// Unlike the forward, long chunks take it too: the two stages would first
// copy every operand (reversed, split), which costs more than the single pass
// loses to them at chunks of 256 and 512.
bool backward_direct(int B, int H, int N, int dk, int dv, int chunk, int dtype, int part_w) {
  if (dtype != RET_BF16) return false;
  if (!ret::fused_supports(dk, dv, chunk) || !ret::fused_supports(part_w, dk, chunk)) return false;
  if (dv % part_w != 0) return false;
  const int64_t heads = static_cast<int64_t>(B) * H;
  if (heads * (dv / 256) < kFusedMinUnits || 2 * heads * (dk / 256) < kFusedMinUnits) return false;
  const int64_t widest = std::max(dk, dv);
  return (static_cast<int64_t>(N) - 1) * widest * 2 + widest * 2 < (int64_t{1} << 30);
}

BackwardPlan plan_backward(int B, int H, int N, int dk, int dv, int chunk, int dtype) {
  BackwardPlan p{};
  p.nparts = dv > kPartWidth ? (dv + kPartWidth - 1) / kPartWidth : 1;
  p.part_w = dv > kPartWidth ? kPartWidth : dv;
  const size_t es = dtype == RET_F32 ? 4 : 2;
  const size_t tok = static_cast<size_t>(B) * H * N;
  const size_t st = static_cast<size_t>(B) * H * dk * dv * sizeof(float);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  p.direct = backward_direct(B, H, N, dk, dv, chunk, dtype, p.part_w);
  if (p.direct) {
    const int64_t heads = static_cast<int64_t>(B) * H;
    p.s_a = take(st);
    p.s_t = take(st);
    p.s_0t = take(st);
    p.s_nt = take(st);
    p.mail = take(std::max(ret::fused_workspace_bytes(heads, dv), ret::fused_workspace_bytes(2 * heads, dk)));
    p.total = off;
    return p;
  }
  p.qf = take(tok * dk * es);
  p.kf = take(tok * dk * es);
  p.dof = take(tok * dv * es);
  p.oa = take(tok * dv * es);
  const bool split = p.nparts > 1;
  p.dos = split ? take(tok * dv * es) : 0;
  p.vs = split ? take(tok * dv * es) : 0;
  p.dofs = split ? take(tok * dv * es) : 0;
  p.vfs = take(tok * dv * es);
  p.kpart = take(tok * dk * es);
  p.s_a = take(st);
  p.s_t = take(st);
  p.s_0t = take(st);
  p.s_nt = take(st);
  size_t cw = plan_chunkwise(B, H, N, dk, dv, chunk, dtype).total;
  for (int q = 0; q < p.nparts; ++q) {
    const int w = std::min(p.part_w, dv - q * p.part_w);
    cw = std::max(cw, plan_chunkwise(B, H, N, w, dk, chunk, dtype).total);
  }
  p.cw_bytes = cw;
  p.cw = take(cw);
  p.total = off;
  return p;
}

// One chunkwise retention as planned: the single-pass kernel, or both stages.
int run_chunkwise(const ChunkPlan& p, const void* q, const void* k, const void* v, void* o, const float* state_in,
                  float* state_out, const Dims& d, int chunk, int dtype, const HeadDecay& decay, const GnArgs& g,
                  char* ws, hipStream_t s, bool accumulate = false) {
  if (p.fused) {
    float* segs = nullptr;
    if (p.nseg > 1) {
      segs = reinterpret_cast<float*>(ws + p.states_bytes);
      // The first segment's workgroups read state_in while the last one's may
      // already write state_out: an aliased state_in is read from a copy.
      const size_t sbytes = static_cast<size_t>(d.B) * d.H * d.dk * d.dv * sizeof(float);
      if (state_in && state_out && overlaps(state_in, sbytes, state_out, sbytes)) {
        float* copy = reinterpret_cast<float*>(ws + p.states_bytes + p.seg_bytes);
        if (ret::copy_device(copy, state_in, sbytes, s) != hipSuccess) return RET_ERR_HIP;
        state_in = copy;
      }
      if (ret::launch_segment_ends(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), state_in, segs,
                                   p.chunks_per_seg, d, chunk, decay, s) != hipSuccess)
        return RET_ERR_HIP;
    }
    return status_of(ret::launch_fused_chunkwise(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                                 static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), state_in,
                                                 state_out, ws, d, chunk, decay, g, accumulate, s, p.chunks_per_seg,
                                                 segs));
  }
  if (launch_states(p, k, v, state_in, state_out, ws, d, chunk, dtype, decay, s) != hipSuccess) return RET_ERR_HIP;
  return status_of(launch_output(p, q, k, v, o, ws, state_in != nullptr, d, chunk, dtype, decay, g, s, accumulate));
}

// One retention for the backward pass: no GroupNorm.
int run_retention(const void* q, const void* k, const void* v, void* o, const float* state_in, float* state_out,
                  const Dims& d, int chunk, int dtype, const HeadDecay& decay, char* cw, hipStream_t s,
                  bool accumulate = false) {
  const ChunkPlan p = plan_chunkwise(d.B, d.H, d.N, d.dk, d.dv, chunk, dtype);
  GnArgs none{};
  return run_chunkwise(p, q, k, v, o, state_in, state_out, d, chunk, dtype, decay, none, cw, s, accumulate);
}

}  // namespace

extern "C" {

int retention_abi_version(void) { return RETENTION_ABI_VERSION; }

const char* retention_status_string(int status) {
  switch (status) {
    case RET_OK: return "ok";
    case RET_ERR_INVALID_ARG: return "invalid argument";
    case RET_ERR_UNSUPPORTED: return "unsupported arguments";
    case RET_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int retention_parallel(const void* q, const void* k, const void* v, const float* gamma_host, void* o, int B, int H,
                       int N, int dk, int dv, int dtype, const retention_gn_t* gn, void* stream) {
  if (!q || !k || !v || !o) return RET_ERR_INVALID_ARG;
  int st = check_sizes(B, H, N, dk, dv, dtype);
  if (st != RET_OK) return st;
  st = check_gamma(gamma_host, H, nullptr);
  if (st != RET_OK) return st;
  GnArgs g;
  st = check_gn(gn, &g);
  if (st != RET_OK) return st;

  if (output_overlaps(q, k, v, o, g.gate, B, H, N, dk, dv, dtype)) return RET_ERR_INVALID_ARG;

  HeadDecay decay;
  check_gamma(gamma_host, H, &decay);
  const Dims d{B, H, N, dk, dv};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == RET_BF16 && ret::mfma_supports(dk, dv)) {
    return status_of(ret::launch_mfma_chunk_out(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                                static_cast<const uint16_t*>(v), nullptr, false,
                                                static_cast<uint16_t*>(o), d, N, decay, g, false, s));
  }
  return status_of(ret::launch_generic_chunk_out(dtype, q, k, v, nullptr, false, o, d, N, decay, g, false, s));
}

size_t retention_chunkwise_workspace_bytes(int B, int H, int N, int dk, int dv, int chunk, int dtype) {
  if (check_sizes(B, H, N, dk, dv, dtype) != RET_OK || chunk <= 0) return 0;
  return plan_chunkwise(B, H, N, dk, dv, effective_chunk(N, chunk), dtype).total;
}

size_t retention_chunk_stages_workspace_bytes(int B, int H, int N, int dk, int dv, int chunk, int dtype) {
  if (check_sizes(B, H, N, dk, dv, dtype) != RET_OK || chunk <= 0) return 0;
  return plan_chunkwise(B, H, N, dk, dv, effective_chunk(N, chunk), dtype, true).total;
}

int retention_chunkwise(const void* q, const void* k, const void* v, const float* gamma_host, void* o, int B, int H,
                        int N, int dk, int dv, int chunk, int dtype, const float* state_in, float* state_out,
                        const retention_gn_t* gn, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o) return RET_ERR_INVALID_ARG;
  GnArgs g;
  ChunkPlan p;
  HeadDecay decay;
  const int st = check_chunkwise(gamma_host, B, H, N, dk, dv, &chunk, dtype, gn, workspace, workspace_bytes, &g, &p,
                                 &decay);
  if (st != RET_OK) return st;
  if (output_overlaps(q, k, v, o, g.gate, B, H, N, dk, dv, dtype)) return RET_ERR_INVALID_ARG;
  const Dims d{B, H, N, dk, dv};
  return run_chunkwise(p, q, k, v, o, state_in, state_out, d, chunk, dtype, decay, g, static_cast<char*>(workspace),
                       static_cast<hipStream_t>(stream));
}

int retention_chunkwise_noalloc(const void* q, const void* k, const void* v, const float* gamma_host, void* o, int B,
                                int H, int N, int dk, int dv, int chunk, int dtype, const float* state_in,
                                float* state_out, const retention_gn_t* gn, void* stream) {
  // Everything is validated before the scratch address is looked up (the
  // first HIP call), exactly as retention_chunkwise validates before launching.
  if (!q || !k || !v || !o || chunk <= 0) return RET_ERR_INVALID_ARG;
  int st = check_sizes(B, H, N, dk, dv, dtype);
  if (st != RET_OK) return st;
  st = check_gamma(gamma_host, H, nullptr);
  if (st != RET_OK) return st;
  GnArgs g;
  st = check_gn(gn, &g);
  if (st != RET_OK) return st;
  const ChunkPlan p = plan_chunkwise(B, H, N, dk, dv, effective_chunk(N, chunk), dtype);
  if (p.total > ret::kScratchBytes) return RET_ERR_UNSUPPORTED;
  if (output_overlaps(q, k, v, o, g.gate, B, H, N, dk, dv, dtype)) return RET_ERR_INVALID_ARG;
  void* ws = nullptr;
  if (p.total > 0 && ret::scratch_pointer(&ws) != hipSuccess) return RET_ERR_HIP;
  return retention_chunkwise(q, k, v, gamma_host, o, B, H, N, dk, dv, chunk, dtype, state_in, state_out, gn, ws,
                             ws ? ret::kScratchBytes : 0, stream);
}

int retention_chunk_states(const void* k, const void* v, const float* gamma_host, int B, int H, int N, int dk,
                           int dv, int chunk, int dtype, const float* state_in, float* state_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!k || !v) return RET_ERR_INVALID_ARG;
  GnArgs g;
  ChunkPlan p;
  HeadDecay decay;
  const int st = check_chunkwise(gamma_host, B, H, N, dk, dv, &chunk, dtype, nullptr, workspace, workspace_bytes, &g,
                                 &p, &decay, true);
  if (st != RET_OK) return st;
  const Dims d{B, H, N, dk, dv};
  return status_of(launch_states(p, k, v, state_in, state_out, static_cast<char*>(workspace), d, chunk, dtype, decay,
                                 static_cast<hipStream_t>(stream)));
}

int retention_chunk_output(const void* q, const void* k, const void* v, const float* gamma_host, void* o, int B,
                           int H, int N, int dk, int dv, int chunk, int dtype, int has_state_in,
                           const retention_gn_t* gn, const void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o) return RET_ERR_INVALID_ARG;
  GnArgs g;
  ChunkPlan p;
  HeadDecay decay;
  const int st = check_chunkwise(gamma_host, B, H, N, dk, dv, &chunk, dtype, gn, workspace, workspace_bytes, &g, &p,
                                 &decay, true);
  if (st != RET_OK) return st;
  if (output_overlaps(q, k, v, o, g.gate, B, H, N, dk, dv, dtype)) return RET_ERR_INVALID_ARG;
  const Dims d{B, H, N, dk, dv};
  return status_of(launch_output(p, q, k, v, o, static_cast<const char*>(workspace), has_state_in != 0, d, chunk,
                                 dtype, decay, g, static_cast<hipStream_t>(stream)));
}

int retention_recurrent_step(const void* q, const void* k, const void* v, const float* gamma_host, float* state,
                             void* o, int B, int H, int dk, int dv, int dtype, const retention_gn_t* gn,
                             void* stream) {
  if (!q || !k || !v || !o || !state) return RET_ERR_INVALID_ARG;
  int st = check_sizes(B, H, 1, dk, dv, dtype);
  if (st != RET_OK) return st;
  st = check_gamma(gamma_host, H, nullptr);
  if (st != RET_OK) return st;
  GnArgs g;
  st = check_gn(gn, &g);
  if (st != RET_OK) return st;
  // (One token: O, Q, K, V and the gate as the N = 1 case; the fp32 state is
  // read and written in place and may share bytes with none of them.)
  if (output_overlaps(q, k, v, o, g.gate, B, H, 1, dk, dv, dtype)) return RET_ERR_INVALID_ARG;
  {
    const size_t es = dtype == RET_F32 ? 4 : 2;
    const size_t sb = static_cast<size_t>(B) * H * dk * dv * sizeof(float);
    const size_t nk = static_cast<size_t>(B) * H * dk * es, nv = static_cast<size_t>(B) * H * dv * es;
    if (overlaps(state, sb, q, nk) || overlaps(state, sb, k, nk) || overlaps(state, sb, v, nv) ||
        overlaps(state, sb, o, nv) || (g.gate && overlaps(state, sb, g.gate, nv)))
      return RET_ERR_INVALID_ARG;
  }
  HeadDecay decay;
  check_gamma(gamma_host, H, &decay);
  return status_of(ret::launch_decode_step(dtype, q, k, v, state, o, B, H, dk, dv, decay, g,
                                           static_cast<hipStream_t>(stream)));
}

int retention_xpos_rotate(const void* q, const void* k, void* q_out, void* k_out, const float* theta_host, int B,
                          int H, int N, int d, long long pos0, int dtype, void* stream) {
  if (!q || !q_out || !theta_host || (k == nullptr) != (k_out == nullptr)) return RET_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || d % 2 != 0 || !valid_dtype(dtype)) return RET_ERR_INVALID_ARG;
  if (d > RETENTION_MAX_DK) return RET_ERR_UNSUPPORTED;
  static_assert(RETENTION_MAX_DK <= 2 * ret::kMaxXposPairs, "xPos angle table");
  if (static_cast<int64_t>(B) * H > INT_MAX) return RET_ERR_INVALID_ARG;
  if (pos0 < 0 || pos0 > (int64_t{1} << 53) - N) return RET_ERR_INVALID_ARG;
  for (int i = 0; i < d / 2; ++i)
    if (!std::isfinite(theta_host[i])) return RET_ERR_INVALID_ARG;
  const size_t esz = dtype == RET_BF16 ? 2 : 4;
  const uintptr_t align = 2 * esz;
  const void* ptrs[4] = {q, k, q_out, k_out};
  for (const void* p : ptrs)
    if (p && reinterpret_cast<uintptr_t>(p) % align != 0) return RET_ERR_INVALID_ARG;
  const size_t n = static_cast<size_t>(B) * H * N * d * esz;
  // Each output is its own input (in place) or shares no byte with any other
  // buffer; the outputs never overlap; an in-place call needs q and k apart.
  if (q_out != q && (overlaps(q_out, n, q, n) || (k && overlaps(q_out, n, k, n)))) return RET_ERR_INVALID_ARG;
  if (k) {
    if (k_out != k && (overlaps(k_out, n, k, n) || overlaps(k_out, n, q, n))) return RET_ERR_INVALID_ARG;
    if (overlaps(k_out, n, q_out, n)) return RET_ERR_INVALID_ARG;
    if ((q_out == q || k_out == k) && overlaps(q, n, k, n)) return RET_ERR_INVALID_ARG;
  }
  return status_of(ret::launch_xpos_rotate(dtype, q, k, q_out, k_out, theta_host, B * H, N, d,
                                           static_cast<int64_t>(pos0), static_cast<hipStream_t>(stream)));
}

size_t retention_chunkwise_backward_workspace_bytes(int B, int H, int N, int dk, int dv, int chunk, int dtype) {
  if (check_sizes(B, H, N, dk, dv, dtype) != RET_OK || chunk <= 0) return 0;
  return plan_backward(B, H, N, dk, dv, effective_chunk(N, chunk), dtype).total;
}

int retention_chunkwise_backward(const void* q, const void* k, const void* v, const void* grad_o,
                                 const float* gamma_host, void* grad_q, void* grad_k, void* grad_v, int B, int H,
                                 int N, int dk, int dv, int chunk, int dtype, const float* state_in,
                                 const float* grad_state_out, float* grad_state_in, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !grad_o || !grad_q || !grad_k || !grad_v || chunk <= 0) return RET_ERR_INVALID_ARG;
  int st = check_sizes(B, H, N, dk, dv, dtype);
  if (st != RET_OK) return st;
  st = check_gamma(gamma_host, H, nullptr);
  if (st != RET_OK) return st;
  // The final-state gradient enters the reverse-time retentions divided by
  // gamma; for a subnormal gamma that quotient overflows float.
  if (grad_state_out) {
    for (int h = 0; h < H; ++h)
      if (gamma_host[h] < FLT_MIN) return RET_ERR_UNSUPPORTED;
  }
  {
    // The gradients are written while the inputs are still read (in place,
    // by other workgroups): no gradient may share bytes with an input or
    // another gradient.
    const size_t es = dtype == RET_F32 ? 4 : 2;
    const size_t tok = static_cast<size_t>(B) * H * N;
    const size_t nk = tok * dk * es, nv = tok * dv * es;
    const void* in[4] = {q, k, v, grad_o};
    const size_t in_n[4] = {nk, nk, nv, nv};
    const void* out[3] = {grad_q, grad_k, grad_v};
    const size_t out_n[3] = {nk, nk, nv};
    for (int i = 0; i < 3; ++i) {
      for (int j = 0; j < 4; ++j)
        if (overlaps(out[i], out_n[i], in[j], in_n[j])) return RET_ERR_INVALID_ARG;
      for (int j = 0; j < i; ++j)
        if (overlaps(out[i], out_n[i], out[j], out_n[j])) return RET_ERR_INVALID_ARG;
    }
  }
  chunk = effective_chunk(N, chunk);
  const BackwardPlan p = plan_backward(B, H, N, dk, dv, chunk, dtype);
  if (!workspace || workspace_bytes < p.total) return RET_ERR_INVALID_ARG;
  HeadDecay decay;
  check_gamma(gamma_host, H, &decay);
  float inv_gamma[RETENTION_MAX_HEADS], fwd_gamma[RETENTION_MAX_HEADS];
  for (int h = 0; h < H; ++h) {
    fwd_gamma[h] = gamma_host[h];
    inv_gamma[h] = static_cast<float>(1.0 / static_cast<double>(gamma_host[h]));
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const size_t es = dtype == RET_F32 ? 4 : 2;
  const int64_t tok = static_cast<int64_t>(B) * H * N;
  const Dims rows{B, H, N, 0, 0};
  auto at = [&](size_t off) { return static_cast<void*>(ws + off); };
  auto st_at = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  auto ok = [](hipError_t e) { return e == hipSuccess; };
  char* cw = ws + p.cw;

  if (p.direct) {
    // The same three retentions as below, on the single-pass kernel reading
    // Q, K, V and dO where they are: reverse order in place of reversed
    // copies, row pitch dv and column offsets in place of the 256-column
    // parts. dV is one launch; each part of dQ and dK is one launch holding
    // both retentions, the first part writing grad_q and grad_k, the later
    // ones adding to them (in fp32, before rounding).
    const int P = p.nparts, pw = p.part_w;
    const int64_t st_part = static_cast<int64_t>(B) * H * pw * dk;  // fp32 elements between state parts
    const GnArgs nogn{};
    auto u16 = [](const void* x) { return static_cast<const uint16_t*>(x); };
    float* s_a = nullptr;
    if (grad_state_out) {
      s_a = st_at(p.s_a);
      if (!ok(ret::launch_state_prep(grad_state_out, s_a, B, H, dk, dv, false, dv, 0, inv_gamma, s)))
        return RET_ERR_HIP;
    }
    float* s_t = grad_state_in ? st_at(p.s_t) : nullptr;
    // dV (and the state gradient): reverse-time retention, query K, key Q, value dO.
    ret::FusedLayout rv;
    rv.reverse = true;
    if (!ok(ret::launch_fused_chunkwise(u16(k), u16(q), u16(grad_o), static_cast<uint16_t*>(grad_v), s_a, s_t,
                                        at(p.mail), Dims{B, H, N, dk, dv}, chunk, decay, nogn, false, s, 0, nullptr,
                                        &rv)))
      return RET_ERR_HIP;
    if (grad_state_in) {
      if (!ok(ret::launch_state_prep(s_t, grad_state_in, B, H, dk, dv, false, dv, 0, fwd_gamma, s)))
        return RET_ERR_HIP;
    }
    float* s_0t = nullptr;
    if (state_in) {
      s_0t = st_at(p.s_0t);
      if (!ok(ret::launch_state_prep(state_in, s_0t, B, H, dk, dv, true, pw, st_part, nullptr, s))) return RET_ERR_HIP;
    }
    float* s_nt = nullptr;
    if (grad_state_out) {
      s_nt = st_at(p.s_nt);
      if (!ok(ret::launch_state_prep(grad_state_out, s_nt, B, H, dk, dv, true, pw, st_part, inv_gamma, s)))
        return RET_ERR_HIP;
    }
    const Dims dd{B, H, N, pw, dk};
    for (int i = 0; i < P; ++i) {
      // dQ part: query dO, key V, value K, starting state S0^T (rows of the part).
      // dK part (reversed time): query V, key dO, value Q, starting state dS_N^T / gamma.
      ret::FusedJob dkj;
      dkj.q = u16(v) + static_cast<int64_t>(i) * pw;
      dkj.k = u16(grad_o) + static_cast<int64_t>(i) * pw;
      dkj.v = u16(q);
      dkj.o = static_cast<uint16_t*>(grad_k);
      dkj.state_in = s_nt ? s_nt + i * st_part : nullptr;
      dkj.reverse = true;
      ret::FusedLayout lq;
      lq.ldq = dv;
      lq.ldk = dv;
      lq.second = &dkj;
      if (!ok(ret::launch_fused_chunkwise(u16(grad_o) + static_cast<int64_t>(i) * pw,
                                          u16(v) + static_cast<int64_t>(i) * pw, u16(k),
                                          static_cast<uint16_t*>(grad_q), s_0t ? s_0t + i * st_part : nullptr,
                                          nullptr, at(p.mail), dd, chunk, decay, nogn, i > 0, s, 0, nullptr, &lq)))
        return RET_ERR_HIP;
    }
    return RET_OK;
  }

  // Operand copies, each source read once: Q and K token-reversed; dO
  // token-reversed whole (the dV retention's value) and, when the dv-wide
  // query/key width of the dQ and dK retentions is cut into parts of at most
  // 256 columns, in parts as it is and token-reversed; V in parts reversed
  // and, when cut, as it is.
  const int P = p.nparts, pw = p.part_w;
  const int64_t part_rows = tok * pw;  // elements between parts (every part but the last is pw wide)
  {
    const ret::SplitTarget tq[1] = {{at(p.qf), dk, 0, true}};
    const ret::SplitTarget tk[1] = {{at(p.kf), dk, 0, true}};
    const ret::SplitTarget to[3] = {{at(p.dof), dv, 0, true}, {at(p.dos), pw, part_rows, false},
                                    {at(p.dofs), pw, part_rows, true}};
    const ret::SplitTarget tv[2] = {{at(p.vfs), pw, part_rows, true}, {at(p.vs), pw, part_rows, false}};
    if (!ok(ret::launch_split_rows(dtype, q, tq, 1, rows, dk, s))) return RET_ERR_HIP;
    if (!ok(ret::launch_split_rows(dtype, k, tk, 1, rows, dk, s))) return RET_ERR_HIP;
    if (!ok(ret::launch_split_rows(dtype, grad_o, to, P > 1 ? 3 : 1, rows, dv, s))) return RET_ERR_HIP;
    if (!ok(ret::launch_split_rows(dtype, v, tv, P > 1 ? 2 : 1, rows, dv, s))) return RET_ERR_HIP;
  }

  // dV (and the state gradient): reverse-time retention with query K, key Q,
  // value dO; the final-state gradient enters as its starting state divided
  // by gamma (the reversed read-out weighs row m' by gamma^(m'+1), the term
  // needs gamma^m').
  float* s_a = nullptr;
  if (grad_state_out) {
    s_a = st_at(p.s_a);
    if (!ok(ret::launch_state_prep(grad_state_out, s_a, B, H, dk, dv, false, dv, 0, inv_gamma, s))) return RET_ERR_HIP;
  }
  float* s_t = grad_state_in ? st_at(p.s_t) : nullptr;
  st = run_retention(at(p.kf), at(p.qf), at(p.dof), at(p.oa), s_a, s_t, Dims{B, H, N, dk, dv}, chunk, dtype, decay,
                     cw, s);
  if (st != RET_OK) return st;
  if (!ok(ret::launch_sum_parts(dtype, at(p.oa), grad_v, rows, dv, 1, 0, true, s))) return RET_ERR_HIP;
  // Its final state T = sum_n gamma^n q_n^T dO_n + gamma^(N-1) dS_N; the state
  // gradient is gamma T.
  if (grad_state_in) {
    if (!ok(ret::launch_state_prep(s_t, grad_state_in, B, H, dk, dv, false, dv, 0, fwd_gamma, s))) return RET_ERR_HIP;
  }

  // Operands of the dQ and dK retentions (copied above).
  const void* dos = P > 1 ? at(p.dos) : grad_o;
  const void* vs = P > 1 ? at(p.vs) : v;
  const void* dofs = P > 1 ? at(p.dofs) : at(p.dof);
  const int64_t st_part = static_cast<int64_t>(B) * H * pw * dk;  // fp32 elements between state parts
  float* s_0t = nullptr;
  if (state_in) {
    s_0t = st_at(p.s_0t);
    if (!ok(ret::launch_state_prep(state_in, s_0t, B, H, dk, dv, true, pw, st_part, nullptr, s))) return RET_ERR_HIP;
  }
  float* s_nt = nullptr;
  if (grad_state_out) {
    s_nt = st_at(p.s_nt);
    if (!ok(ret::launch_state_prep(grad_state_out, s_nt, B, H, dk, dv, true, pw, st_part, inv_gamma, s)))
      return RET_ERR_HIP;
  }

  auto part = [&](const void* base, int i) {
    return static_cast<const void*>(static_cast<const char*>(base) + static_cast<size_t>(i) * part_rows * es);
  };
  // The parts' results are summed in place: the first part writes, the later
  // ones add (in fp32, before rounding) to what is there.
  for (int i = 0; i < P; ++i) {
    const int w = std::min(pw, dv - i * pw);
    const Dims dd{B, H, N, w, dk};
    // dQ part: query dO, key V, value K, starting state S0^T (rows of the part).
    st = run_retention(part(dos, i), part(vs, i), k, grad_q, s_0t ? s_0t + i * st_part : nullptr, nullptr, dd, chunk,
                       dtype, decay, cw, s, i > 0);
    if (st != RET_OK) return st;
    // dK part (reversed time): query V, key dO, value Q, starting state dS_N^T / gamma.
    st = run_retention(part(at(p.vfs), i), part(dofs, i), at(p.qf), at(p.kpart), s_nt ? s_nt + i * st_part : nullptr,
                       nullptr, dd, chunk, dtype, decay, cw, s, i > 0);
    if (st != RET_OK) return st;
  }
  return status_of(ret::launch_sum_parts(dtype, at(p.kpart), grad_k, rows, dk, 1, 0, true, s));
}

}  // extern "C"
