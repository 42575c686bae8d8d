// Host side of the C ABI declared in include/kairos.h: argument validation
// (complete before anything is enqueued), workspace layout, and the launch
// sequence of each entry point on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <new>

#include "kairos.h"
#include "common.hpp"

#include "launch.hpp"

using namespace kairos;

// Execution context of layer calls (kairos_context_create): a side stream of
// the device it was created on, the events that fork work onto it and join
// it back, and the device's compute-unit count.  Owned by the caller; the
// mutex orders the record / wait pairs of calls that share the context.
struct kairos_context_t {
  int device = -1;
  int cus = 0;
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, gdn = nullptr;
  std::mutex mu;
};

namespace kairos {

// Count of the n gate pairs with alpha outside (0, 1] or beta outside
// [0, beta_max] (NaN counts as outside) into *count, overwritten
// (csrc/gates_check.hip).
hipError_t launch_gate_check(const float* alpha, const float* beta, long n, float beta_max, uint32_t* count,
                             hipStream_t stream);

// Scratch array of kairos_gdn_fwd_noalloc, the workspace of callers that
// cannot allocate device memory.  Each device the library runs on holds its
// own copy until the process ends.  Host code never uses the array's name as
// an address (on the host it is only a stand-in for the symbol): the device
// address of each device's copy is resolved once, with that device current,
// and kept in noalloc_scratch_ptr.  Every no-alloc call on a device shares
// its copy, so such calls must not overlap on one device.
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
constexpr int kMaxNoallocDevices = 64;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];
void* noalloc_scratch_ptr[kMaxNoallocDevices];
std::mutex noalloc_scratch_mu;

}  // namespace kairos

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;   // bound on any tensor's element count
constexpr size_t kWsAlign = 256;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

// operand format of the windowed branches' q and k: 0 bf16, 1 E4M3 codes,
// 2 E2M1 codes (two per byte); the last two come with per-block scales
int qk_format(int window_qk) {
  return window_qk == KAIROS_FP8_E4M3 ? 1 : window_qk == KAIROS_FP4_E2M1 ? 2 : 0;
}
size_t qk_bytes(int qf, size_t n) { return qf == 2 ? n / 2 : qf == 1 ? n : 2 * n; }

// Quantisation blocks per frame when they restart at every frame (0: the
// call's token order), and scale entries per (b, h) of one quantised tensor.
int blocks_per_frame(const kairos_hlta_desc* d) {
  return qk_format(d->window_qk) != 0 && d->qk_blocks == KAIROS_QK_BLOCKS_FRAMES ? (d->L + 63) / 64 : 0;
}
size_t scale_blocks(const kairos_hlta_desc* d) {
  const int nbf = blocks_per_frame(d);
  return nbf > 0 ? (size_t)((d->g.T + d->L - 1) / d->L) * nbf : (size_t)(d->g.T + 63) / 64;
}

// Parts of a layer call's key ring: with RoPE and dilation > 1 the two
// windowed branches rotate keys at different positions, and the ring keeps
// each branch's rotated keys ([2][B][R][L][H][d]); otherwise one part.
int ring_key_parts(const kairos_hlta_desc* d) { return d->rope_base > 0.f && d->dilation > 1 ? 2 : 1; }

// Ring layout: V [B][R][L][H][d] bf16; keys in ring_key_parts parts, each the
// key rows [B][R][L][H][row] (bf16, or codes) and, for quantised keys, their
// block scales [B][H][R][nbf] fp32 after the rows (256-byte aligned).
struct RingLayout {
  size_t v_bytes, k_rows, k_scales, k_part, k_bytes;
};
RingLayout ring_layout(const kairos_hlta_desc* d) {
  RingLayout r{};
  const int qf = qk_format(d->window_qk);
  const size_t toks = (size_t)d->g.B * d->ring_frames * d->L * d->g.H;
  r.v_bytes = toks * d->g.dk * 2;
  r.k_rows = qk_bytes(qf, toks * d->g.dk);
  const size_t ns = qf != 0 ? (size_t)d->g.B * d->g.H * d->ring_frames * blocks_per_frame(d) * 4 : 0;
  r.k_scales = ns > 0 ? align_up(r.k_rows) : 0;
  r.k_part = ns > 0 ? align_up(r.k_scales + ns) : r.k_rows;
  r.k_bytes = r.k_part * ring_key_parts(d);
  return r;
}

int check_gdn_desc(const kairos_gdn_desc* d) {
  if (!d) return KAIROS_ERR_NULL;
  if (d->B < 1 || d->H < 1 || d->T < 0) return KAIROS_ERR_SHAPE;
  if (d->dk != d->dv) return KAIROS_ERR_SHAPE;
  if (d->dk != 32 && d->dk != 64 && d->dk != 128) return KAIROS_ERR_SHAPE;
  if (d->chunk != 64) return KAIROS_ERR_SHAPE;
  if (d->io != KAIROS_F32 && d->io != KAIROS_BF16) return KAIROS_ERR_DTYPE;
  if (d->io == KAIROS_BF16 && d->dk == 32) return KAIROS_ERR_UNSUPPORTED;
  const int64_t n = (int64_t)d->B * d->T * d->H * d->dk;
  if (n > kMaxElems) return KAIROS_ERR_SHAPE;
  // one workgroup per (b, h) of the fp32 path; the chunk kernels address the
  // rows of a 64-token chunk by 32-bit byte offsets and count their
  // workgroups in 32-bit integers
  if ((int64_t)d->B * d->H > INT32_MAX) return KAIROS_ERR_SHAPE;
  if (d->io == KAIROS_BF16) {
    const int64_t tok_bytes = (int64_t)d->H * d->dk * 2;
    if (63 * tok_bytes + d->dk * 2 >= ((int64_t)1 << 32)) return KAIROS_ERR_SHAPE;
    if ((int64_t)d->B * d->H * ((d->T + 63) / 64) > INT32_MAX) return KAIROS_ERR_SHAPE;
  }
  return KAIROS_OK;
}

int check_hlta_desc(const kairos_hlta_desc* d, bool layer) {
  if (!d) return KAIROS_ERR_NULL;
  int st = check_gdn_desc(&d->g);
  if (st != KAIROS_OK) return st;
  if (d->g.io != KAIROS_BF16) return KAIROS_ERR_DTYPE;
  if (d->g.dk != 128) return KAIROS_ERR_UNSUPPORTED;
  if (d->L < 1 || d->window < 1 || d->dilation < 1 || d->frame_offset < 0 || d->ring_frames < 0)
    return KAIROS_ERR_SHAPE;
  // the window kernel addresses a key block's rows as 32-bit offsets (row x H x 256 bytes)
  if (d->g.H > 65536) return KAIROS_ERR_SHAPE;
  if (d->window_kind != KAIROS_WINDOW_CAUSAL && d->window_kind != KAIROS_WINDOW_CENTERED)
    return KAIROS_ERR_SHAPE;
  if (d->window_kind == KAIROS_WINDOW_CENTERED && d->ring_frames > 0) return KAIROS_ERR_UNSUPPORTED;
  if (!(d->rope_base >= 0.f) || !(d->rope_base < 3.0e38f)) return KAIROS_ERR_SHAPE;
  if (d->qk_blocks != KAIROS_QK_BLOCKS_TOKENS && d->qk_blocks != KAIROS_QK_BLOCKS_FRAMES) return KAIROS_ERR_SHAPE;
  if (d->window_qk != KAIROS_BF16 && d->window_qk != KAIROS_FP8_E4M3 && d->window_qk != KAIROS_FP4_E2M1)
    return KAIROS_ERR_DTYPE;
  // a streamed rollout quantises exactly as one run over the whole sequence
  // only if no quantisation block mixes two calls' tokens
  if (d->window_qk != KAIROS_BF16 && d->ring_frames > 0 && d->qk_blocks != KAIROS_QK_BLOCKS_FRAMES)
    return KAIROS_ERR_UNSUPPORTED;
  // group positions (frame / dil) * L + L and token indices must fit in int32
  const int64_t frames = (d->g.T + d->L - 1) / d->L;
  if ((d->frame_offset + frames + 1) * (int64_t)d->L >= ((int64_t)1 << 30)) return KAIROS_ERR_SHAPE;
  if ((int64_t)d->window >= ((int64_t)1 << 30)) return KAIROS_ERR_SHAPE;
  if (d->ring_frames > 0) {
    if (d->g.T % d->L != 0) return KAIROS_ERR_SHAPE;
    const int64_t need = (int64_t)d->dilation * ((d->window - 1 + d->L - 1) / d->L);
    if (d->ring_frames < need) return KAIROS_ERR_SHAPE;
  }
  (void)layer;
  return KAIROS_OK;
}

// Layer workspace: GDN chunk data, o_gdn, the parked partial result of the
// window kernel (a row per query) and its log-sum-exp (one per query), and
// the windowed operands of each branch (E4M3 codes + scales, or with RoPE the
// rotated q, k; the second set only when RoPE gives DSWA its own operands).
struct HltaWs {
  size_t gdn, o_gdn, ypart, ylse;
  size_t q1, k1, qs1, ks1;   // first-branch operands (codes / rotated bf16), scales (codes)
  size_t q2, k2, qs2, ks2;   // second-branch operands (RoPE with dilation > 1)
  bool has1, has2;
  size_t total;
};

size_t gdn_ws_bytes(const kairos_gdn_desc* d) {
  return d->io == KAIROS_BF16 ? gdn_chunk_workspace(d->B, d->T, d->H, d->dk) : 0;
}

HltaWs hlta_ws_layout(const kairos_hlta_desc* d) {
  HltaWs w{};
  const size_t n = (size_t)d->g.B * d->g.T * d->g.H * d->g.dk;
  const int qf = qk_format(d->window_qk);
  const bool fp8 = qf != 0;
  const bool rope = d->rope_base > 0.f;
  const size_t nsc = fp8 ? (size_t)d->g.B * d->g.H * scale_blocks(d) * 4 : 0;
  size_t off = 0;
  w.gdn = off;
  off += align_up(gdn_ws_bytes(&d->g));
  w.o_gdn = off;
  off += align_up(n * 2);
  w.ypart = off;
  off += align_up(n * 4);
  w.ylse = off;
  off += align_up(n / d->g.dk * 4);
  w.has1 = fp8 || rope;
  w.has2 = rope && d->dilation > 1;
  for (int set = 0; set < 2; ++set) {
    if (!(set == 0 ? w.has1 : w.has2)) continue;
    size_t* q = set == 0 ? &w.q1 : &w.q2;
    size_t* k = set == 0 ? &w.k1 : &w.k2;
    size_t* qs = set == 0 ? &w.qs1 : &w.qs2;
    size_t* ks = set == 0 ? &w.ks1 : &w.ks2;
    *q = off;
    off += align_up(qk_bytes(qf, n));
    *k = off;
    off += align_up(qk_bytes(qf, n));
    *qs = off;
    off += align_up(nsc);
    *ks = off;
    off += align_up(nsc);
  }
  w.total = off;
  return w;
}

// RoPE of q and k of one branch into the workspace (bf16 or E4M3 + scales).
hipError_t rope_branch(const kairos_hlta_desc* d, int dil, const void* q, const void* k, void* qo,
                       void* ko, float* qs, float* ks, hipStream_t s) {
  OperandArgs r;
  memset(&r, 0, sizeof(r));
  r.x[0] = (const uint16_t*)q;
  r.x[1] = (const uint16_t*)k;
  r.out[0] = qo;
  r.out[1] = ko;
  r.scales[0] = qs;
  r.scales[1] = ks;
  r.nt = 2;
  r.B = d->g.B;
  r.T = d->g.T;
  r.H = d->g.H;
  r.L = d->L;
  r.dil = dil;
  r.nblk = (int)scale_blocks(d);
  r.nbf = blocks_per_frame(d);
  r.frame_offset = (long)d->frame_offset;
  return launch_rope(r, d->g.dk, (double)d->rope_base, qk_format(d->window_qk), s);
}

int check_gdn_ptrs(const kairos_gdn_desc* d, const void* q, const void* k, const void* v,
                   const float* alpha, const float* beta, const float* state_in, const void* out,
                   const float* state_out) {
  if (d->T > 0 && (!q || !k || !v || !alpha || !beta || !out)) return KAIROS_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(state_in) ||
      !aligned16(state_out))
    return KAIROS_ERR_ALIGN;
  if (((uintptr_t)alpha & 3u) || ((uintptr_t)beta & 3u)) return KAIROS_ERR_ALIGN;
  const size_t esz = d->io == KAIROS_F32 ? 4 : 2;
  const size_t nx = (size_t)d->B * d->T * d->H * d->dk * esz;
  const size_t ng = (size_t)d->B * d->T * d->H * 4;
  const size_t ns = (size_t)d->B * d->H * d->dk * d->dv * 4;
  if (overlaps(out, nx, q, nx) || overlaps(out, nx, k, nx) || overlaps(out, nx, v, nx) ||
      overlaps(out, nx, alpha, ng) || overlaps(out, nx, beta, ng) || overlaps(out, nx, state_in, ns) ||
      overlaps(out, nx, state_out, ns))
    return KAIROS_ERR_ALIAS;
  if (state_out && state_out != state_in &&
      (overlaps(state_out, ns, state_in, ns) || overlaps(state_out, ns, q, nx) ||
       overlaps(state_out, ns, k, nx) || overlaps(state_out, ns, v, nx) ||
       overlaps(state_out, ns, alpha, ng) || overlaps(state_out, ns, beta, ng)))
    return KAIROS_ERR_ALIAS;
  return KAIROS_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? KAIROS_OK : KAIROS_ERR_HIP; }

void fill_win_args(WinArgs& a, const kairos_hlta_desc* d) {
  memset(&a, 0, sizeof(a));
  a.B = d->g.B;
  a.T = d->g.T;
  a.H = d->g.H;
  a.L = d->L;
  a.F = (d->g.T + d->L - 1) / d->L;
  a.w = d->window;
  a.dil = d->dilation;
  a.R = d->ring_frames;
  a.nblk = (int)scale_blocks(d);
  a.nbf = blocks_per_frame(d);
  a.centered = d->window_kind == KAIROS_WINDOW_CENTERED ? 1 : 0;
  a.frame_offset = (long)d->frame_offset;
}

// Whether a layer call may use its context's side stream: always when the
// side stream is idle or eager; when it belongs to a graph capture (it was
// forked into one and stays in it until that capture ends), only if the
// caller's stream is part of the same capture.  Otherwise (another thread's
// capture holds the side stream) the call runs on the caller's stream alone.
bool side_usable(const kairos_context_t* c, hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone, ss = hipStreamCaptureStatusNone;
  unsigned long long cid = 0, sid = 0;
  if (hipStreamGetCaptureInfo(c->side, &ss, &sid) != hipSuccess) return false;
  if (ss == hipStreamCaptureStatusNone) return true;
  if (hipStreamGetCaptureInfo(s, &cs, &cid) != hipSuccess) return false;
  return ss == hipStreamCaptureStatusActive && cs == hipStreamCaptureStatusActive && cid == sid;
}

// Device address of the current device's copy of the scratch array,
// resolved on the first no-alloc call on that device.
int noalloc_scratch(void** p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return KAIROS_ERR_HIP;
  if (dev >= kMaxNoallocDevices) return KAIROS_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(noalloc_scratch_mu);
  if (!noalloc_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KAIROS_ERR_HIP;
    noalloc_scratch_ptr[dev] = ptr;
  }
  *p = noalloc_scratch_ptr[dev];
  return KAIROS_OK;
}

// The launch sequence of kairos_gdn_fwd once the arguments are checked.
int gdn_fwd_launch(const kairos_gdn_desc* desc, const void* q, const void* k, const void* v,
                   const float* alpha, const float* beta, const float* state_in, void* out,
                   float* state_out, void* workspace, hipStream_t s);

// Whether a layer call runs its GDN branch beside the window kernel (the
// window epilogue then leaves the windowed sum in fp32 and a combine kernel
// adds the gated GDN output), rather than before it: only when both grids
// fit on the device at once (two workgroups per compute unit), i.e. when the
// window kernel alone would leave compute units idle, as for one streamed
// frame.  On larger calls the extra fp32 round trip and the scan's share of
// the compute units cost more than the overlap saves (measured: one 1560-
// token frame at H 24 -10%; 21 frames +10%; the B4 16 x 3600 FP8 layer +4%).
bool overlap_gdn(const kairos_hlta_desc* d, const kairos_context_t* c) {
  if (!c || c->cus <= 0 || d->g.dk != 128) return false;
  const long win = window_workgroups(d->g.B, d->g.T, d->g.H, d->L);
  const long gdn = (long)d->g.B * d->g.H * (d->g.dk / (16 * gdn_chunk_waves(d->g.B, d->g.H, d->g.dk)));
  return win + gdn <= 2L * c->cus;
}

int gdn_fwd_launch(const kairos_gdn_desc* desc, const void* q, const void* k, const void* v,
                   const float* alpha, const float* beta, const float* state_in, void* out,
                   float* state_out, void* workspace, hipStream_t s) {
  if (desc->io == KAIROS_F32)
    return hip_status(launch_gdn_f32((const float*)q, (const float*)k, (const float*)v, alpha, beta,
                                     state_in, (float*)out, state_out, desc->B, desc->T, desc->H,
                                     desc->dk, s));
  return hip_status(launch_gdn_chunk((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                                     alpha, beta, state_in, (uint16_t*)out, state_out, desc->B,
                                     desc->T, desc->H, desc->dk, 0, workspace, s));
}

}  // namespace

extern "C" {

const char* kairos_status_string(int status) {
  switch (status) {
    case KAIROS_OK: return "ok";
    case KAIROS_ERR_NULL: return "null pointer";
    case KAIROS_ERR_SHAPE: return "invalid shape";
    case KAIROS_ERR_DTYPE: return "unsupported dtype";
    case KAIROS_ERR_ALIGN: return "misaligned buffer";
    case KAIROS_ERR_ALIAS: return "overlapping buffers";
    case KAIROS_ERR_UNSUPPORTED: return "unsupported combination";
    case KAIROS_ERR_WORKSPACE: return "workspace missing or too small";
    case KAIROS_ERR_HIP: return "HIP runtime error";
    case KAIROS_ERR_RANGE: return "input values out of range";
    default: return "unknown status";
  }
}

int kairos_version(void) { return 202; }

int kairos_gdn_workspace_size(const kairos_gdn_desc* desc, size_t* bytes) {
  if (!bytes) return KAIROS_ERR_NULL;
  const int st = check_gdn_desc(desc);
  if (st != KAIROS_OK) return st;
  *bytes = gdn_ws_bytes(desc);
  return KAIROS_OK;
}

int kairos_hlta_workspace_size(const kairos_hlta_desc* desc, size_t* bytes) {
  if (!bytes) return KAIROS_ERR_NULL;
  const int st = check_hlta_desc(desc, true);
  if (st != KAIROS_OK) return st;
  *bytes = hlta_ws_layout(desc).total;
  return KAIROS_OK;
}

int kairos_hlta_ring_size(const kairos_hlta_desc* desc, size_t* k_bytes, size_t* v_bytes) {
  if (!k_bytes || !v_bytes) return KAIROS_ERR_NULL;
  const int st = check_hlta_desc(desc, true);
  if (st != KAIROS_OK) return st;
  const RingLayout rl = ring_layout(desc);
  *k_bytes = rl.k_bytes;
  *v_bytes = rl.v_bytes;
  return KAIROS_OK;
}

int kairos_hlta_ring_frames_required(const kairos_hlta_desc* desc, int32_t* frames) {
  if (!desc || !frames) return KAIROS_ERR_NULL;
  if (desc->L < 1 || desc->window < 1 || desc->dilation < 1) return KAIROS_ERR_SHAPE;
  *frames = (int32_t)((int64_t)desc->dilation * ((desc->window - 1 + desc->L - 1) / desc->L));
  return KAIROS_OK;
}

int kairos_gdn_fwd(const kairos_gdn_desc* desc, const void* q, const void* k, const void* v,
                   const float* alpha, const float* beta, const float* state_in, void* out,
                   float* state_out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_gdn_desc(desc);
  if (st != KAIROS_OK) return st;
  st = check_gdn_ptrs(desc, q, k, v, alpha, beta, state_in, out, state_out);
  if (st != KAIROS_OK) return st;
  const size_t need = gdn_ws_bytes(desc);
  if (need > 0 && (!workspace || workspace_bytes < need)) return KAIROS_ERR_WORKSPACE;
  if (((uintptr_t)workspace & (kWsAlign - 1)) != 0) return KAIROS_ERR_ALIGN;
  const size_t nx = (size_t)desc->B * desc->T * desc->H * desc->dk * (desc->io == KAIROS_F32 ? 4 : 2);
  if (overlaps(workspace, need, out, nx) || overlaps(workspace, need, q, nx) ||
      overlaps(workspace, need, k, nx) || overlaps(workspace, need, v, nx) ||
      overlaps(workspace, need, state_out, (size_t)desc->B * desc->H * desc->dk * desc->dv * 4))
    return KAIROS_ERR_ALIAS;
  return gdn_fwd_launch(desc, q, k, v, alpha, beta, state_in, out, state_out, workspace,
                        (hipStream_t)stream);
}

int kairos_gdn_fwd_noalloc(const kairos_gdn_desc* desc, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, const float* state_in, void* out,
                           float* state_out, void* stream) {
  int st = check_gdn_desc(desc);
  if (st != KAIROS_OK) return st;
  st = check_gdn_ptrs(desc, q, k, v, alpha, beta, state_in, out, state_out);
  if (st != KAIROS_OK) return st;
  const size_t need = gdn_ws_bytes(desc);
  if (need > kNoallocScratchBytes) return KAIROS_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    st = noalloc_scratch(&ws);
    if (st != KAIROS_OK) return st;
  }
  return gdn_fwd_launch(desc, q, k, v, alpha, beta, state_in, out, state_out, ws, (hipStream_t)stream);
}

int kairos_window_fwd(const kairos_hlta_desc* desc, int32_t dilation, const void* q, const void* k,
                      const void* v, const float* q_scales, const float* k_scales,
                      const void* k_ring, const void* v_ring, void* out, void* stream) {
  int st = check_hlta_desc(desc, false);
  if (st != KAIROS_OK) return st;
  if (dilation < 1) return KAIROS_ERR_SHAPE;
  if (desc->ring_frames > 0) {
    const int64_t need = (int64_t)dilation * ((desc->window - 1 + desc->L - 1) / desc->L);
    if (desc->ring_frames < need) return KAIROS_ERR_SHAPE;
  }
  const int qf = qk_format(desc->window_qk);
  const bool fp8 = qf != 0;
  if (desc->rope_base != 0.f) return KAIROS_ERR_UNSUPPORTED;
  // external scales come from the token-order quantisers; a ring of quantised
  // keys exists only inside the layer call
  if (fp8 && (desc->qk_blocks != KAIROS_QK_BLOCKS_TOKENS || desc->ring_frames > 0)) return KAIROS_ERR_UNSUPPORTED;
  if (desc->g.T == 0) return KAIROS_OK;
  if (!q || !k || !v || !out) return KAIROS_ERR_NULL;
  if (fp8 && (!q_scales || !k_scales)) return KAIROS_ERR_NULL;
  if (!fp8 && (q_scales || k_scales)) return KAIROS_ERR_UNSUPPORTED;
  if (desc->ring_frames > 0 && (!k_ring || !v_ring)) return KAIROS_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(k_ring) ||
      !aligned16(v_ring))
    return KAIROS_ERR_ALIGN;
  const size_t n = (size_t)desc->g.B * desc->g.T * desc->g.H * desc->g.dk;
  const size_t nqk = qk_bytes(qf, n);
  const size_t nring = (size_t)desc->g.B * desc->ring_frames * desc->L * desc->g.H * desc->g.dk * 2;
  if (overlaps(out, 2 * n, q, nqk) || overlaps(out, 2 * n, k, nqk) || overlaps(out, 2 * n, v, 2 * n) ||
      overlaps(out, 2 * n, k_ring, nring) || overlaps(out, 2 * n, v_ring, nring))
    return KAIROS_ERR_ALIAS;
  WinArgs a;
  fill_win_args(a, desc);
  a.dil = dilation;
  a.q = q;
  a.k = k;
  a.v = (const uint16_t*)v;
  a.q_scales = q_scales;
  a.k_scales = k_scales;
  a.k_ring = (const uint16_t*)k_ring;
  a.v_ring = (const uint16_t*)v_ring;
  a.out = (uint16_t*)out;
  return hip_status(launch_window(a, qf, false, (hipStream_t)stream));
}

int kairos_hlta_window_fwd(const kairos_hlta_desc* desc, const void* q, const void* k,
                           const void* v, const float* q_scales, const float* k_scales,
                           const void* o_gdn, const float* gate_logits, const void* k_ring,
                           const void* v_ring, void* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  int st = check_hlta_desc(desc, true);
  if (st != KAIROS_OK) return st;
  // the parked partial result (a row per query) and its log-sum-exp (one per query)
  const size_t nws = (size_t)desc->g.B * desc->g.T * desc->g.H * (desc->g.dk + 1) * 4;
  const int qf = qk_format(desc->window_qk);
  const bool fp8 = qf != 0;
  if (desc->rope_base != 0.f) return KAIROS_ERR_UNSUPPORTED;
  if (fp8 && (desc->qk_blocks != KAIROS_QK_BLOCKS_TOKENS || desc->ring_frames > 0)) return KAIROS_ERR_UNSUPPORTED;
  if (desc->g.T == 0) return KAIROS_OK;
  if (!q || !k || !v || !o_gdn || !gate_logits || !out) return KAIROS_ERR_NULL;
  if (fp8 && (!q_scales || !k_scales)) return KAIROS_ERR_NULL;
  if (!fp8 && (q_scales || k_scales)) return KAIROS_ERR_UNSUPPORTED;
  if (desc->ring_frames > 0 && (!k_ring || !v_ring)) return KAIROS_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_gdn) || !aligned16(out) ||
      !aligned16(k_ring) || !aligned16(v_ring))
    return KAIROS_ERR_ALIGN;
  const size_t n = (size_t)desc->g.B * desc->g.T * desc->g.H * desc->g.dk;
  const size_t nqk = qk_bytes(qf, n);
  const size_t nring = (size_t)desc->g.B * desc->ring_frames * desc->L * desc->g.H * desc->g.dk * 2;
  if (overlaps(out, 2 * n, q, nqk) || overlaps(out, 2 * n, k, nqk) || overlaps(out, 2 * n, v, 2 * n) ||
      overlaps(out, 2 * n, o_gdn, 2 * n) || overlaps(out, 2 * n, k_ring, nring) ||
      overlaps(out, 2 * n, v_ring, nring))
    return KAIROS_ERR_ALIAS;
  if (!workspace || workspace_bytes < nws) return KAIROS_ERR_WORKSPACE;
  if (((uintptr_t)workspace & (kWsAlign - 1)) != 0) return KAIROS_ERR_ALIGN;
  if (overlaps(workspace, nws, out, 2 * n) || overlaps(workspace, nws, q, nqk) ||
      overlaps(workspace, nws, k, nqk) || overlaps(workspace, nws, v, 2 * n) ||
      overlaps(workspace, nws, o_gdn, 2 * n))
    return KAIROS_ERR_ALIAS;
  WinArgs a;
  fill_win_args(a, desc);
  a.ypart = (float*)workspace;
  a.ylse = (float*)((uint8_t*)workspace + n * 4);
  a.q = q;
  a.k = k;
  a.v = (const uint16_t*)v;
  a.q_scales = q_scales;
  a.k_scales = k_scales;
  a.k_ring = (const uint16_t*)k_ring;
  a.v_ring = (const uint16_t*)v_ring;
  a.o_gdn = (const uint16_t*)o_gdn;
  a.gates = gate_logits;
  a.out = (uint16_t*)out;
  return hip_status(launch_window(a, qf, true, (hipStream_t)stream));
}

int kairos_context_create(kairos_context* ctx) {
  if (!ctx) return KAIROS_ERR_NULL;
  *ctx = nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return KAIROS_ERR_HIP;
  kairos_context_t* c = new (std::nothrow) kairos_context_t;
  if (!c) return KAIROS_ERR_HIP;
  c->device = dev;
  bool ok = hipDeviceGetAttribute(&c->cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&c->fork, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&c->join, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&c->gdn, hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    kairos_context_destroy(c);
    return KAIROS_ERR_HIP;
  }
  *ctx = c;
  return KAIROS_OK;
}

int kairos_context_destroy(kairos_context ctx) {
  if (!ctx) return KAIROS_OK;
  bool ok = true;
  if (ctx->side) ok &= hipStreamDestroy(ctx->side) == hipSuccess;
  for (hipEvent_t ev : {ctx->fork, ctx->join, ctx->gdn})
    if (ev) ok &= hipEventDestroy(ev) == hipSuccess;
  delete ctx;
  return ok ? KAIROS_OK : KAIROS_ERR_HIP;
}

int kairos_hlta_fwd(const kairos_hlta_desc* desc, const void* q, const void* k, const void* v,
                    const float* alpha, const float* beta, const float* gate_logits,
                    const float* state_in, void* k_ring, void* v_ring, void* out, float* state_out,
                    void* workspace, size_t workspace_bytes, kairos_context ctx, void* stream) {
  int st = check_hlta_desc(desc, true);
  if (st != KAIROS_OK) return st;
  if (ctx) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return KAIROS_ERR_HIP;
    if (dev != ctx->device) return KAIROS_ERR_UNSUPPORTED;
  }
  st = check_gdn_ptrs(&desc->g, q, k, v, alpha, beta, state_in, out, state_out);
  if (st != KAIROS_OK) return st;
  if (!gate_logits) return KAIROS_ERR_NULL;
  if (desc->ring_frames > 0 && (!k_ring || !v_ring)) return KAIROS_ERR_NULL;
  if (!aligned16(k_ring) || !aligned16(v_ring)) return KAIROS_ERR_ALIGN;
  const HltaWs ws = hlta_ws_layout(desc);
  if (ws.total > 0 && (!workspace || workspace_bytes < ws.total)) return KAIROS_ERR_WORKSPACE;
  if (((uintptr_t)workspace & (kWsAlign - 1)) != 0) return KAIROS_ERR_ALIGN;
  const size_t n = (size_t)desc->g.B * desc->g.T * desc->g.H * desc->g.dk;
  const RingLayout rl = ring_layout(desc);
  const size_t nring = rl.v_bytes, nkring = rl.k_bytes;
  if (overlaps(k_ring, nkring, v_ring, nring) || overlaps(k_ring, nkring, out, 2 * n) ||
      overlaps(v_ring, nring, out, 2 * n) || overlaps(k_ring, nkring, k, 2 * n) ||
      overlaps(v_ring, nring, v, 2 * n) || overlaps(k_ring, nkring, q, 2 * n) ||
      overlaps(workspace, ws.total, k_ring, nkring) || overlaps(workspace, ws.total, v_ring, nring) ||
      overlaps(workspace, ws.total, out, 2 * n) ||
      overlaps(workspace, ws.total, q, 2 * n) || overlaps(workspace, ws.total, k, 2 * n) ||
      overlaps(workspace, ws.total, v, 2 * n))
    return KAIROS_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  const int B = desc->g.B, T = desc->g.T, H = desc->g.H, D = desc->g.dk;
  uint8_t* wsb = (uint8_t*)workspace;
  uint16_t* o_gdn = (uint16_t*)(wsb + ws.o_gdn);
  // Two schedules, both ordered as one stream for the caller:
  // * overlapped: the GDN branch runs on the side stream beside the operand
  //   pre-passes and the window kernel, whose epilogue leaves the windowed
  //   sum in fp32; a combine kernel adds the gated GDN output;
  // * otherwise: the GDN branch first, the operand pre-passes on the side
  //   stream once its prep kernel is done (both are bandwidth-bound; the
  //   scan is not), the window kernel's epilogue adds the GDN output.
  kairos_context_t* sd = T > 0 ? ctx : nullptr;
  std::unique_lock<std::mutex> lk;
  if (sd) {
    lk = std::unique_lock<std::mutex>(sd->mu);
    if (!side_usable(sd, s)) {
      lk.unlock();
      sd = nullptr;
    }
  }
  const bool ovl = overlap_gdn(desc, sd);
  if (sd && !ovl && !ws.has1 && !ws.has2) {            // one stream is enough
    lk.unlock();
    sd = nullptr;
  }
  hipError_t e;
  if (ovl) {
    if (hipEventRecord(sd->fork, s) != hipSuccess || hipStreamWaitEvent(sd->side, sd->fork, 0) != hipSuccess)
      return KAIROS_ERR_HIP;
    e = launch_gdn_chunk((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, alpha, beta,
                         state_in, o_gdn, state_out, B, T, H, D, 0, wsb + ws.gdn, sd->side);
    if (e != hipSuccess || hipEventRecord(sd->gdn, sd->side) != hipSuccess) return KAIROS_ERR_HIP;
  } else {
    e = launch_gdn_chunk((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, alpha, beta,
                         state_in, o_gdn, state_out, B, T, H, D, 0, wsb + ws.gdn, s,
                         sd ? sd->fork : nullptr);
    if (e != hipSuccess) return KAIROS_ERR_HIP;
  }
  if (T == 0) return KAIROS_OK;
  const hipStream_t so = (sd && !ovl) ? sd->side : s;   // stream of the operand pre-passes
  if (so != s && hipStreamWaitEvent(so, sd->fork, 0) != hipSuccess) return KAIROS_ERR_HIP;
  WinArgs a;
  fill_win_args(a, desc);
  a.v = (const uint16_t*)v;
  a.k_ring = (const uint16_t*)k_ring;
  a.v_ring = (const uint16_t*)v_ring;
  if (desc->ring_frames > 0 && rl.k_scales > 0) a.ks_ring = (const float*)((const uint8_t*)k_ring + rl.k_scales);
  a.o_gdn = ovl ? nullptr : o_gdn;
  a.gates = gate_logits;
  a.ypart = (float*)(wsb + ws.ypart);
  a.ylse = (float*)(wsb + ws.ylse);
  a.out = (uint16_t*)out;
  const int qf = qk_format(desc->window_qk);
  const bool fp8 = qf != 0;
  const bool rope = desc->rope_base > 0.f;
  a.q = q;
  a.k = k;
  if (ws.has1) {
    void* q1 = wsb + ws.q1;
    void* k1 = wsb + ws.k1;
    float* qs1 = fp8 ? (float*)(wsb + ws.qs1) : nullptr;
    float* ks1 = fp8 ? (float*)(wsb + ws.ks1) : nullptr;
    if (rope) {
      e = rope_branch(desc, 1, q, k, q1, k1, qs1, ks1, so);
    } else {
      const int nbf = blocks_per_frame(desc);
      e = launch_block_quant((const uint16_t*)q, (uint8_t*)q1, qs1, B, T, H, D, qf, so, desc->L, nbf);
      if (e == hipSuccess)
        e = launch_block_quant((const uint16_t*)k, (uint8_t*)k1, ks1, B, T, H, D, qf, so, desc->L, nbf);
    }
    if (e != hipSuccess) return KAIROS_ERR_HIP;
    a.q = q1;
    a.k = k1;
    a.q_scales = qs1;
    a.k_scales = ks1;
  }
  if (ws.has2) {
    void* q2 = wsb + ws.q2;
    void* k2 = wsb + ws.k2;
    float* qs2 = fp8 ? (float*)(wsb + ws.qs2) : nullptr;
    float* ks2 = fp8 ? (float*)(wsb + ws.ks2) : nullptr;
    e = rope_branch(desc, desc->dilation, q, k, q2, k2, qs2, ks2, so);
    if (e != hipSuccess) return KAIROS_ERR_HIP;
    a.q2 = q2;
    a.k2 = k2;
    a.q_scales2 = qs2;
    a.k_scales2 = ks2;
    if (desc->ring_frames > 0) {
      a.k_ring2 = (const uint16_t*)((const uint8_t*)k_ring + rl.k_part);
      if (rl.k_scales > 0) a.ks_ring2 = (const float*)((const uint8_t*)k_ring + rl.k_part + rl.k_scales);
    }
  }
  if (so != s && (hipEventRecord(sd->join, so) != hipSuccess || hipStreamWaitEvent(s, sd->join, 0) != hipSuccess))
    return KAIROS_ERR_HIP;
  e = launch_window(a, qf, true, s);
  if (e != hipSuccess) return KAIROS_ERR_HIP;
  if (ovl) {
    if (hipStreamWaitEvent(s, sd->gdn, 0) != hipSuccess) return KAIROS_ERR_HIP;
    e = launch_hlta_combine(a.ypart, o_gdn, gate_logits, (uint16_t*)out, B, T, H, s);
    if (e != hipSuccess) return KAIROS_ERR_HIP;
  }
  if (desc->ring_frames > 0) {
    // the ring keeps the keys the windowed branches read: with RoPE the
    // rotated ones (each branch's, at its own positions; absolute positions
    // make a rotated key valid in every later call)
    const int F = T / desc->L, R = desc->ring_frames;
    const long fo = (long)desc->frame_offset;
    const int krow = (int)qk_bytes(qf, D);
    e = launch_ring_copy(v, v_ring, B, F, desc->L, H, 2 * D, fo, R, s);
    for (int part = 0; part < ring_key_parts(desc) && e == hipSuccess; ++part) {
      // part 0: the first branch's keys; part 1: the second branch's own keys
      uint8_t* dst = (uint8_t*)k_ring + part * rl.k_part;
      e = launch_ring_copy(part ? a.k2 : a.k, dst, B, F, desc->L, H, krow, fo, R, s);
      if (e == hipSuccess && rl.k_scales > 0)
        e = launch_ring_copy_scales(part ? a.k_scales2 : a.k_scales, (float*)(dst + rl.k_scales), B * H, F,
                                    blocks_per_frame(desc), fo, R, s);
    }
    if (e != hipSuccess) return KAIROS_ERR_HIP;
  }
  return KAIROS_OK;
}

int kairos_gdn_prologue(const kairos_gdn_desc* desc, int32_t flags, const void* k_in,
                        const float* alpha_logits, const float* beta_logits, const void* q_in,
                        const void* v_in, void* k_out, float* alpha_out, float* beta_out,
                        void* q_out, void* v_out, void* stream) {
  int st = check_gdn_desc(desc);
  if (st != KAIROS_OK) return st;
  if (flags & ~(KAIROS_PROLOGUE_NORMALIZE_Q | KAIROS_PROLOGUE_LITERAL_EQ6))
    return KAIROS_ERR_UNSUPPORTED;
  const bool nq = (flags & KAIROS_PROLOGUE_NORMALIZE_Q) != 0;
  const bool lit = (flags & KAIROS_PROLOGUE_LITERAL_EQ6) != 0;
  if (!nq && (q_in || q_out)) return KAIROS_ERR_UNSUPPORTED;
  if (!lit && (v_in || v_out)) return KAIROS_ERR_UNSUPPORTED;
  if (desc->T == 0) return KAIROS_OK;
  if (!k_in || !k_out || !alpha_logits || !beta_logits || !alpha_out || !beta_out)
    return KAIROS_ERR_NULL;
  if (nq && (!q_in || !q_out)) return KAIROS_ERR_NULL;
  if (lit && (!v_in || !v_out)) return KAIROS_ERR_NULL;
  if (!aligned16(k_in) || !aligned16(k_out) || !aligned16(q_in) || !aligned16(q_out) ||
      !aligned16(v_in) || !aligned16(v_out))
    return KAIROS_ERR_ALIGN;
  if (((uintptr_t)alpha_logits | (uintptr_t)beta_logits | (uintptr_t)alpha_out |
       (uintptr_t)beta_out) & 3u)
    return KAIROS_ERR_ALIGN;
  const long rows = (long)desc->B * desc->T * desc->H;
  const size_t nx = (size_t)rows * desc->dk * (desc->io == KAIROS_F32 ? 4 : 2);
  const size_t ng = (size_t)rows * 4;
  // outputs[i] may coincide exactly with inputs[i] and overlap nothing else
  const void* ins[5] = {k_in, alpha_logits, beta_logits, q_in, v_in};
  const void* outs[5] = {k_out, alpha_out, beta_out, q_out, v_out};
  const size_t sz[5] = {nx, ng, ng, nx, nx};
  for (int i = 0; i < 5; ++i) {
    if (!outs[i]) continue;
    for (int j = 0; j < 5; ++j) {
      if (j != i && overlaps(outs[i], sz[i], ins[j], sz[j])) return KAIROS_ERR_ALIAS;
      if (j != i && overlaps(outs[i], sz[i], outs[j], sz[j])) return KAIROS_ERR_ALIAS;
    }
    if (outs[i] != ins[i] && overlaps(outs[i], sz[i], ins[i], sz[i])) return KAIROS_ERR_ALIAS;
  }
  PrologueArgs a;
  a.k_in = k_in;
  a.q_in = q_in;
  a.v_in = v_in;
  a.za = alpha_logits;
  a.zb = beta_logits;
  a.k_out = k_out;
  a.q_out = q_out;
  a.v_out = v_out;
  a.alpha = alpha_out;
  a.beta = beta_out;
  a.rows = rows;
  return hip_status(launch_gdn_prologue(a, desc->dk, desc->io == KAIROS_F32, nq, lit,
                                        (hipStream_t)stream));
}

int kairos_rope(const kairos_hlta_desc* desc, int32_t dilation, const void* x, void* out,
                float* scales, void* stream) {
  int st = check_hlta_desc(desc, false);
  if (st != KAIROS_OK) return st;
  if (!(desc->rope_base > 0.f) || dilation < 1) return KAIROS_ERR_SHAPE;
  const int qf = qk_format(desc->window_qk);
  const bool fp8 = qf != 0;
  if (!fp8 && scales) return KAIROS_ERR_UNSUPPORTED;
  if (fp8 && desc->qk_blocks != KAIROS_QK_BLOCKS_TOKENS) return KAIROS_ERR_UNSUPPORTED;
  if (desc->g.T == 0) return KAIROS_OK;
  if (!x || !out || (fp8 && !scales)) return KAIROS_ERR_NULL;
  if (!aligned16(x) || !aligned16(out) || ((uintptr_t)scales & 3u)) return KAIROS_ERR_ALIGN;
  const size_t n = (size_t)desc->g.B * desc->g.T * desc->g.H * desc->g.dk;
  const size_t ns = (size_t)desc->g.B * desc->g.H * ((desc->g.T + 63) / 64) * 4;
  if (fp8 ? overlaps(out, qk_bytes(qf, n), x, 2 * n) : (out != x && overlaps(out, 2 * n, x, 2 * n)))
    return KAIROS_ERR_ALIAS;
  if (overlaps(scales, ns, x, 2 * n) || overlaps(scales, ns, out, qk_bytes(qf, n)))
    return KAIROS_ERR_ALIAS;
  OperandArgs r;
  memset(&r, 0, sizeof(r));
  r.x[0] = (const uint16_t*)x;
  r.out[0] = out;
  r.scales[0] = scales;
  r.nt = 1;
  r.B = desc->g.B;
  r.T = desc->g.T;
  r.H = desc->g.H;
  r.L = desc->L;
  r.dil = dilation;
  r.nblk = (desc->g.T + 63) / 64;
  r.frame_offset = (long)desc->frame_offset;
  return hip_status(launch_rope(r, desc->g.dk, (double)desc->rope_base, qf, (hipStream_t)stream));
}

namespace {

int block_quantize(const void* x_bf16, uint8_t* codes, float* scales, int32_t B, int32_t T, int32_t H,
                   int32_t d, int fmt, void* stream) {
  if (B < 1 || H < 1 || T < 0) return KAIROS_ERR_SHAPE;
  if (d != 32 && d != 64 && d != 128) return KAIROS_ERR_SHAPE;
  if ((int64_t)B * T * H * d > kMaxElems || B > 65535 || (H + 3) / 4 > 65535) return KAIROS_ERR_SHAPE;
  if (T == 0) return KAIROS_OK;
  if (!x_bf16 || !codes || !scales) return KAIROS_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(codes) || ((uintptr_t)scales & 3u)) return KAIROS_ERR_ALIGN;
  const size_t n = (size_t)B * T * H * d;
  const size_t nc = qk_bytes(fmt, n);
  const size_t ns = (size_t)B * H * ((T + 63) / 64) * 4;
  if (overlaps(codes, nc, x_bf16, 2 * n) || overlaps(scales, ns, x_bf16, 2 * n) ||
      overlaps(scales, ns, codes, nc))
    return KAIROS_ERR_ALIAS;
  return hip_status(launch_block_quant((const uint16_t*)x_bf16, codes, scales, B, T, H, d, fmt,
                                       (hipStream_t)stream));
}

}  // namespace

int kairos_gdn_check_gates(const float* alpha, const float* beta, int32_t B, int32_t T, int32_t H,
                           float beta_max, uint32_t* count, void* stream) {
  if (B < 1 || H < 1 || T < 0 || !(beta_max >= 0.f)) return KAIROS_ERR_SHAPE;
  const int64_t n = (int64_t)B * T * H;
  if (n > kMaxElems) return KAIROS_ERR_SHAPE;
  if (!count || (n > 0 && (!alpha || !beta))) return KAIROS_ERR_NULL;
  if (((uintptr_t)count & 3u) != 0 || !aligned16(alpha) || !aligned16(beta)) return KAIROS_ERR_ALIGN;
  if (overlaps(count, 4, alpha, (size_t)n * 4) || overlaps(count, 4, beta, (size_t)n * 4)) return KAIROS_ERR_ALIAS;
  return hip_status(launch_gate_check(alpha, beta, (long)n, beta_max, count, (hipStream_t)stream));
}

int kairos_fp8_quantize(const void* x_bf16, uint8_t* codes, float* scales, int32_t B, int32_t T,
                        int32_t H, int32_t d, void* stream) {
  return block_quantize(x_bf16, codes, scales, B, T, H, d, 1, stream);
}

int kairos_fp4_quantize(const void* x_bf16, uint8_t* codes, float* scales, int32_t B, int32_t T,
                        int32_t H, int32_t d, void* stream) {
  return block_quantize(x_bf16, codes, scales, B, T, H, d, 2, stream);
}

}  // extern "C"
