// Sliding-window (SWA) and dilated sliding-window (DSWA) softmax attention on
// gfx950, causal or centred, with the fused per-head sigmoid branch-gate
// epilogue of the hybrid layer.
//
// Operation (Kairos paper, arXiv 2606.16533 HTML v3, Sec. 2.2.2):
//   SWA (Eq. 7, causal reading):  o_i = sum_{i-w < j <= i} softmax_j(q_i.k_j / sqrt(d)) v_j
//   SWA (Eq. 7 as printed, centred): keys |j - i| <= r, r = floor(w / 2)
//   DSWA (Eq. 8): SWA over the sequence rearranged so that frames with equal
//   (absolute frame index mod dilation) are contiguous.  Nothing is moved in
//   memory: with f the absolute frame of a token, its group is f mod dil and
//   its position inside the group's sequence is p = (f / dil) * L + offset;
//   keys of query i are the tokens of its group with p_i - w < p_j <= p_i.
//   SWA is the same map with dil = 1, so one code path serves both.
//   Both window forms are one band [p_i - back, min(p_i + fwd, p_last)] in
//   group positions (causal: back = w - 1, fwd = 0; centred: back = fwd = r;
//   p_last is the group's last position that exists in the call).
//   Hybrid epilogue: y = sig(z_swa) o_swa + sig(z_dswa) o_dswa + sig(z_gdn) o_gdn.
//
// Work decomposition: one workgroup (4 waves) per (batch, head, frame,
// 128-query tile); query tiles never straddle a frame, so each tile has one
// contiguous key range per branch in group-position space.  Keys are walked
// in blocks of at most 64 positions: with bf16 Q/K, 64 consecutive group
// positions (rows of one block may come from two frames, or from the ring of
// a streamed rollout); with quantised Q/K in frames of at least 64 tokens,
// blocks stop at frame ends and at the call's 64-token quantisation blocks,
// so each block has one key scale, applied together with the query's.  Each
// block's K and V rows go from global memory straight into double-buffered
// LDS, token-major, each lane of a load writing 16 bytes of one row.  Each
// wave owns 32 queries: S^T = K Q^T on 32x32 matrix-core tiles with Q held
// in registers, an online softmax in exp2 form (one query per lane, the row
// reduction is within the lane plus one exchange with lane ^ 32), then
// O^T += V^T P^T with P taken straight from the score registers and the V^T
// operands read with the transposing LDS read.  With E4M3 (E2M1) Q/K the
// score product uses the 32x32x64 f8f6f4 instruction; P V stays bf16.
//
// Key order inside a 32-key tile: the score tile's row r maps to key
// pi(r) = 16 j + 8 g + 4 h + i for r = 16 j + 8 h + 4 g + i (bits g and h
// swapped).  With that order the 8 score registers a lane feeds into one
// P V product step are 8 consecutive keys.
//
// The running maximum is only raised when a block's maximum exceeds it by
// more than 8 (log2 units): probabilities then stay <= 2^8, which is exact
// to rescale away at the end, and the O rescale is skipped in almost every
// block.  Most blocks first form their probabilities against the running
// maximum as it stands and check only their sum; the block maximum is taken
// (and the block formed again) only when that sum exceeds 2^32.
//
// Quantised Q/K in frames of at least one block run three workgroups per CU
// (three waves per SIMD), bf16 Q/K and shorter frames two, so that one wave's
// softmax arithmetic overlaps another's matrix products.  To fit, the hybrid
// kernel parks the finished first branch (gated, normalised, fp32) in a
// workspace row per query and adds it back in the epilogue.  When both
// branches score the same q and k (no RoPE) and the dilation exceeds 1, the
// query's own frame is scored once for both: SWA's other frames are parked
// with their log-sum-exp, the own frame's softmax state is merged into that
// row and then carried on over DSWA's other frames (a softmax over disjoint
// key sets is the log-sum-exp weighted mix of the per-set results).
#include "common.hpp"
#include "launch.hpp"

namespace kairos {

constexpr int WD = 128;          // head dimension
constexpr int BQ = 128;          // queries per workgroup
constexpr int BK = 64;           // keys per block
constexpr int KST = WD + 16;     // bf16 K LDS row stride (elements): 16 mod 32
constexpr int K8ST = WD;         // E4M3 K LDS row stride (bytes), 16-byte units XOR-swizzled
constexpr int K4ST = WD / 2;     // E2M1 K LDS row stride (bytes, two codes per byte), swizzled

// Q/K operand formats (template parameter QF)
constexpr int QF_BF16 = 0, QF_FP8 = 1, QF_FP4 = 2;
// bytes of one token's row of q or k in memory
__device__ __forceinline__ constexpr int qk_row_bytes(int qf) {
  return qf == QF_FP4 ? WD / 2 : qf == QF_FP8 ? WD : 2 * WD;
}
constexpr int VST = 2 * WD;      // V LDS row stride (bytes), 16-byte units XOR-swizzled

// Unpadded K (E4M3) and V rows in LDS: 16-byte unit u of row r is stored in
// slot u ^ f(r).  Measured on gfx950, both keep their reads (the 32-row
// operand reads of K, the transposed 4-row reads of V) as fast as padded rows
// (V faster), with fewer loads per block.
__device__ __forceinline__ constexpr int k8_swz(int r) { return (r >> 1) & 7; }
// E2M1 K rows: 4 units; a 16-lane group reads 16 rows at one unit position,
// which land in 16 distinct 16-byte slots of 256 bytes
__device__ __forceinline__ constexpr int k4_swz(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ constexpr int v_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
constexpr float RESCALE_SLACK = 8.f;
// a lane's block sum above this (2^32) sends the block to the maximum and
// rescale path; a wave stops forming blocks against the running maximum
// alone after SPEC_TRIES such blocks in one branch
constexpr float SPEC_LIMIT = 4294967296.f;
constexpr int SPEC_TRIES = 4;

typedef short wshort4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void wlds_void;

// Transposed LDS read of 16-bit elements (see the lane map in the gated
// delta rule scan): lane i of a 16-lane group gets column c(i/4) + i%4 of
// rows k0..k0+3 when lane s addresses row k0 + s/4, columns c(s%4)...
__device__ __forceinline__ uint2 win_read_tr(const uint16_t* p) {
  const wshort4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((wshort4 __attribute__((address_space(3)))*)(p));
  return __builtin_bit_cast(uint2, r);
}
__device__ __forceinline__ void to_lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (wlds_void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void to_lds4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (wlds_void*)lds, 4, 0, 0);
}
__device__ __forceinline__ void win_wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// LDS layout of one key block: K rows (E4M3 128 bytes and E2M1 64 bytes,
// 16-byte units XOR-swizzled; bf16 256 bytes + 32 padding), V rows (256
// bytes, swizzled), and fp32 key scales for quantised keys in frames shorter
// than a block.  A block of U 16-byte units per row is U loads of 64 lanes
// (lane l of load m fills unit 64 m + l).
template <int QF, bool SHORTL>
struct WinGeom {
  static constexpr bool FP8 = QF != QF_BF16;                  // block-quantised codes + key scales
  static constexpr int KU = QF == QF_FP4 ? K4ST / 16 : QF == QF_FP8 ? K8ST / 16 : KST * 2 / 16;   // units per K row (4 / 8 / 18)
  static constexpr int VU = VST / 16;                         // units per V row (16)
  static constexpr int KBYTES = BK * KU * 16;
  static constexpr int VBYTES = BK * VU * 16;
  // per-key scales travel with the block only where blocks may straddle a
  // quantisation block (frames shorter than a block); otherwise a block has
  // one scale, read directly
  static constexpr bool SCL = FP8 && SHORTL;
  static constexpr int NLOAD = KU + VU + (SCL ? 1 : 0);       // loads per block (all waves)
  static constexpr int NJ = (NLOAD + 3) / 4;                  // loads per wave
};

// Position -> source row map of one branch for one workgroup.
struct KeyMap {
  int L, dil, res, R, frame_offset;
};

// First element of the frame at sub-frame index n of the group: a frame of
// the call, or (frames before the call) a ring slot.  row_bytes: bytes of one
// token's row of this head.
__device__ __forceinline__ const uint8_t* frame_base(const KeyMap& km, const uint8_t* x,
                                                     const uint8_t* ring, int row_bytes, int b,
                                                     int h, int T, int H, int n) {
  const int f = n * km.dil + km.res;                       // absolute frame
  if (f >= km.frame_offset)
    return x + (((size_t)b * T + (size_t)(f - km.frame_offset) * km.L) * H + h) * (size_t)row_bytes;
  return ring + (((size_t)b * km.R + f % km.R) * km.L * (size_t)H + h) * (size_t)row_bytes;
}

// Key scales of the frame at sub-frame index n of the group, with blocks
// restarting at every frame (nbf per frame): the call's scales, or for frames
// before the call the ring's (slot f mod R).  kscale / kring_scale: this
// branch's arrays; the result indexes by row / 64.
__device__ __forceinline__ const float* frame_scales(const KeyMap& km, const float* kscale,
                                                     const float* kring_scale, int b, int h, int H,
                                                     int nblk, int nbf, int n) {
  const int f = n * km.dil + km.res;                       // absolute frame
  if (f >= km.frame_offset) return kscale + ((size_t)b * H + h) * nblk + (size_t)(f - km.frame_offset) * nbf;
  return kring_scale + (((size_t)b * H + h) * km.R + f % km.R) * nbf;
}

// Key range of one branch for one query tile, in group-position space.
struct BranchRange {
  KeyMap km;
  int pq0;      // group position of query row m = 0 of the frame
  int p_lo, p_hi, nb;
  int back, fwd;  // reach of a query's window before / after its own position
  int p_last;     // last group position present in the call
  bool own_k;     // keys from the second-branch operands (a.k2, a.k_scales2)
};

__device__ __forceinline__ BranchRange branch_range(const WinArgs& a, int dil, int f, int m_first,
                                                    int m_last) {
  BranchRange r;
  const int f_abs = (int)a.frame_offset + f;
  r.km.L = a.L;
  r.km.dil = dil;
  r.km.res = f_abs % dil;
  r.km.R = a.R;
  r.km.frame_offset = (int)a.frame_offset;
  r.pq0 = (f_abs / dil) * a.L;
  const int f_avail = (int)a.frame_offset - a.R > 0 ? (int)a.frame_offset - a.R : 0;
  const int f1 = f_avail + (((r.km.res - f_avail % dil) % dil) + dil) % dil;   // first frame of the group
  const int p_avail = (f1 / dil) * a.L;
  // last frame of the group inside the call (only the call's last frame may be partial)
  const int f_end = (int)a.frame_offset + a.F - 1;
  const int f_lastg = f_end - (f_end - r.km.res) % dil;
  const int len_last = min(a.L, a.T - (f_lastg - (int)a.frame_offset) * a.L);
  r.p_last = (f_lastg / dil) * a.L + len_last - 1;
  r.back = a.centered ? a.w / 2 : a.w - 1;
  r.fwd = a.centered ? a.w / 2 : 0;
  const int lo = r.pq0 + m_first - r.back;
  r.p_lo = lo > p_avail ? lo : p_avail;
  r.p_hi = min(r.pq0 + m_last + r.fwd, r.p_last);
  r.nb = (r.p_hi - r.p_lo + BK) / BK;
  r.own_k = false;
  return r;
}

// Combine a value with the one of lane ^ 32: the two halves of the wave swap
// registers inside the vector unit (no LDS round trip); each lane receives
// its own value and its partner's, in some order.
__device__ __forceinline__ float max_with_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// key offset inside a 64-key block of score register r of tile kt (lane group g)
__device__ __forceinline__ constexpr int key_of(int kt, int r, int g) {
  return 32 * kt + 16 * (r / 8) + 8 * g + 4 * ((r / 4) & 1) + (r & 3);
}

// Per-lane query state shared by the branch loops.
struct QueryCtx {
  int b, h, mq, mw_lo, mw_hi, krow, ql, g, wave;
  bool active;     // the wave has at least one query row inside the frame
  float cq;
  int k8o[2][2];   // E4M3 K: byte offset of this lane's operand halves (step s, half) in a 32-row tile
  int k4o[2];      // E2M1 K: byte offset of this lane's operand (step s) in a 32-row tile
  int vo[4][2];    // V: byte offset of this lane's transposed reads (feature tile dt, rows +0 / +4)
};

// One LDS buffer of a key block (pointers into separate __shared__ variables).
struct WinBuf {
  uint8_t* K;
  uint16_t* V;
  float* sk;
};

// This wave's share of a block's loads: entry j is load e = wave + 4 j of
// the block (K loads, then V loads, then the E4M3 scales); per lane the key
// row and byte offset inside the row, and the source address.
template <int QF, bool SHORTL>
struct WinLoads {
  const uint8_t* src[WinGeom<QF, SHORTL>::NJ];
  uint32_t inc[WinGeom<QF, SHORTL>::NJ];   // source step of a block inside one frame (64 rows)
  // blocks inside one frame (aligned quantised blocks): wave-uniform address
  // of the block's first K and V rows and per-lane offsets from them
  const uint8_t* kb;
  const uint8_t* vb;
  uint32_t off[WinGeom<QF, SHORTL>::NJ];
};

// Key row and byte offset inside the row of this lane's load j (computed
// where the addresses are rebuilt, so they hold no registers in between).
template <int QF, bool SHORTL>
__device__ __forceinline__ void slot_rowcol(int j, int wave, int& row, int& col) {
  using G = WinGeom<QF, SHORTL>;
  const int lane = threadIdx.x % 64;
  const int e = (wave & 3) + 4 * j;   // wave < 4: lets the compiler fold the slot kinds
  int U, upr;
  if (e < G::KU) { U = 64 * e + lane; upr = G::KU; }
  else if (e < G::KU + G::VU) { U = 64 * (e - G::KU) + lane; upr = G::VU; }
  else { U = lane; upr = 1; }                      // scales: one per key
  row = U / upr;
  const int u = U % upr;                           // LDS slot of the row
  if (e < G::KU)
    col = QF == QF_FP4 ? (u ^ k4_swz(row)) * 16
        : QF == QF_FP8 ? (u ^ k8_swz(row)) * 16 : (u % 16) * 16;   // bf16: padding copies a unit
  else if (e < G::KU + G::VU) col = (u ^ v_swz(row)) * 16;
  else col = 0;
}

template <int QF, bool SHORTL>
__device__ __forceinline__ void win_load_setup(WinLoads<QF, SHORTL>& ld, int wave, int H) {
  using G = WinGeom<QF, SHORTL>;
#pragma unroll
  for (int j = 0; j < G::NJ; ++j) {
    const int e = (wave & 3) + 4 * j;   // wave < 4: lets the compiler fold the slot kinds
    ld.inc[j] = e < G::KU ? (uint32_t)BK * H * qk_row_bytes(QF)
              : e < G::KU + G::VU ? (uint32_t)BK * H * WD * 2 : 4u;    // scales: next 64-token block
  }
}

// Source addresses of the block at group position pb (sub-frame n0, offset
// m0): positions past p_hi clamp to p_hi (masked out; clamping keeps loads in
// bounds and values finite).
template <int QF, bool SHORTL>
__device__ __forceinline__ void win_block_addrs(WinLoads<QF, SHORTL>& ld, const WinArgs& a, const BranchRange& br,
                                                int b, int h, int wave, int pb, int n0, int m0) {
  using G = WinGeom<QF, SHORTL>;
  constexpr int KROW = qk_row_bytes(QF);
  const KeyMap& km = br.km;
  const int p_hi = br.p_hi;
  const uint8_t* kx = reinterpret_cast<const uint8_t*>(br.own_k ? a.k2 : a.k);
  const uint8_t* kring = reinterpret_cast<const uint8_t*>(br.own_k && a.k_ring2 ? a.k_ring2 : a.k_ring);
  const uint8_t* vx = reinterpret_cast<const uint8_t*>(a.v);
  const uint8_t* vring = reinterpret_cast<const uint8_t*>(a.v_ring);
  const int L = km.L;
  const size_t rs_k = (size_t)a.H * KROW, rs_v = (size_t)a.H * WD * 2;
  const uint8_t* k0 = nullptr;
  const uint8_t* k1 = nullptr;
  const uint8_t* v0 = nullptr;
  const uint8_t* v1 = nullptr;
  if (!SHORTL) {
    const int n1 = min(n0 + 1, p_hi / L);
    k0 = frame_base(km, kx, kring, KROW, b, h, a.T, a.H, n0);
    k1 = frame_base(km, kx, kring, KROW, b, h, a.T, a.H, n1);
    v0 = frame_base(km, vx, vring, 2 * WD, b, h, a.T, a.H, n0);
    v1 = frame_base(km, vx, vring, 2 * WD, b, h, a.T, a.H, n1);
  }
#pragma unroll
  for (int j = 0; j < G::NJ; ++j) {
    const int e = (wave & 3) + 4 * j;   // wave < 4: lets the compiler fold the slot kinds
    if (e >= G::NLOAD) continue;
    int row, col;
    slot_rowcol<QF, SHORTL>(j, wave, row, col);
    const int d = min(pb + row, p_hi) - pb;
    const int m = m0 + d;
    int n, mm;
    if (SHORTL) { n = n0 + m / L; mm = m - (m / L) * L; }
    else { n = n0 + (m >= L ? 1 : 0); mm = m >= L ? m - L : m; }
    if (e < G::KU) {
      const uint8_t* base = SHORTL ? frame_base(km, kx, kring, KROW, b, h, a.T, a.H, n) : (n == n0 ? k0 : k1);
      ld.src[j] = base + (size_t)mm * rs_k + col;
    } else if (e < G::KU + G::VU) {
      const uint8_t* base = SHORTL ? frame_base(km, vx, vring, 2 * WD, b, h, a.T, a.H, n) : (n == n0 ? v0 : v1);
      ld.src[j] = base + (size_t)mm * rs_v + col;
    } else {
      const float* ksc = br.own_k ? a.k_scales2 : a.k_scales;
      if (a.nbf > 0) {       // blocks restart at every frame; ring frames have their own scales
        const float* ksr = br.own_k && a.ks_ring2 ? a.ks_ring2 : a.ks_ring;
        ld.src[j] = reinterpret_cast<const uint8_t*>(frame_scales(km, ksc, ksr, b, h, a.H, a.nblk, a.nbf, n) + mm / 64);
      } else {               // token-order blocks (no ring): rows are tokens of the call
        const int tok = (n * km.dil + km.res - km.frame_offset) * L + mm;
        ld.src[j] = reinterpret_cast<const uint8_t*>(ksc + ((size_t)b * a.H + h) * a.nblk + tok / 64);
      }
    }
  }
}

// Addresses of an aligned block (inside sub-frame n0, from row m0): rows past
// the block's last valid row dmax repeat it (masked out), so every row stays
// inside the frame and the call.
template <int QF, bool SHORTL>
__device__ __forceinline__ void win_block_addrs_al(WinLoads<QF, SHORTL>& ld, const WinArgs& a,
                                                   const BranchRange& br, int b, int h, int wave, int n0,
                                                   int m0, int dmax) {
  using G = WinGeom<QF, SHORTL>;
  constexpr int KROW = qk_row_bytes(QF);
  const KeyMap& km = br.km;
  const uint8_t* kx = reinterpret_cast<const uint8_t*>(br.own_k ? a.k2 : a.k);
  const uint8_t* kring = reinterpret_cast<const uint8_t*>(br.own_k && a.k_ring2 ? a.k_ring2 : a.k_ring);
  const uint8_t* vx = reinterpret_cast<const uint8_t*>(a.v);
  const uint8_t* vring = reinterpret_cast<const uint8_t*>(a.v_ring);
  const uint32_t rs_k = (uint32_t)a.H * KROW, rs_v = (uint32_t)a.H * WD * 2;
  ld.kb = frame_base(km, kx, kring, KROW, b, h, a.T, a.H, n0) + (size_t)m0 * rs_k;
  ld.vb = frame_base(km, vx, vring, 2 * WD, b, h, a.T, a.H, n0) + (size_t)m0 * rs_v;
#pragma unroll
  for (int j = 0; j < G::NJ; ++j) {
    const int e = (wave & 3) + 4 * j;   // wave < 4: lets the compiler fold the slot kinds
    if (e >= G::NLOAD) continue;
    int row, col;
    slot_rowcol<QF, SHORTL>(j, wave, row, col);
    ld.off[j] = (uint32_t)min(row, dmax) * (e < G::KU ? rs_k : rs_v) + (uint32_t)col;
  }
}

template <int QF, bool SHORTL>
__device__ __forceinline__ void win_issue_al(const WinLoads<QF, SHORTL>& ld, const WinBuf& bf, int wave) {
  using G = WinGeom<QF, SHORTL>;
#pragma unroll
  for (int j = 0; j < G::NJ; ++j) {
    const int e = (wave & 3) + 4 * j;   // wave < 4: lets the compiler fold the slot kinds
    if (e < G::KU) to_lds16(ld.kb + ld.off[j], bf.K + 1024 * e);
    else if (e < G::KU + G::VU) to_lds16(ld.vb + ld.off[j], reinterpret_cast<uint8_t*>(bf.V) + 1024 * (e - G::KU));
  }
}

template <int QF, bool SHORTL>
__device__ __forceinline__ void win_issue(const WinLoads<QF, SHORTL>& ld, const WinBuf& bf, int wave) {
  using G = WinGeom<QF, SHORTL>;
#pragma unroll
  for (int j = 0; j < G::NJ; ++j) {
    const int e = (wave & 3) + 4 * j;   // wave < 4: lets the compiler fold the slot kinds
    if (e < G::KU) to_lds16(ld.src[j], bf.K + 1024 * e);
    else if (e < G::KU + G::VU) to_lds16(ld.src[j], reinterpret_cast<uint8_t*>(bf.V) + 1024 * (e - G::KU));
    else if (e < G::NLOAD) to_lds4(ld.src[j], bf.sk);
  }
}

// Scores S^T of one key block from buffer cb (two 32-key tiles; lane: query
// ql, key key_of(kt, r, g)), per-key scales applied unless ALIGN, and keys
// outside the lane's window at -inf.  The lane's query sees the keys at group
// positions [hi - wl + 1, hi].
template <int QF, bool ALIGN>
__device__ __forceinline__ void win_scores(const WinBuf& cb, const QueryCtx& qc, int hi, int wl, int pb,
                                           int size, bool full, const bf16x8 (&qf)[8],
                                           const i32x8 (&q8f)[2], f32x16 (&S)[2]) {
  constexpr bool FP8 = QF != QF_BF16;
  S[0] = f32x16{};
  S[1] = f32x16{};
  if (!FP8) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const uint16_t* Ks = reinterpret_cast<const uint16_t*>(cb.K) + (32 * kt + qc.krow) * KST;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        S[kt] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(Ks + 16 * s + 8 * qc.g)), qf[s], S[kt]);
    }
  } else {
    // all four quantised operands are read before the first product; the
    // products alternate between the two score tiles.  E4M3: 32 codes (two
    // 16-byte reads) per lane and step; E2M1: 32 codes in one 16-byte read
    // (the instruction reads the low four registers of the operand).
    i32x8 ka[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (QF == QF_FP4) {
          const uint4 lo = *reinterpret_cast<const uint4*>(cb.K + 32 * kt * K4ST + qc.k4o[s]);
          ka[kt][s] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
        } else {
          const uint8_t* K8 = cb.K + 32 * kt * K8ST;
          const uint4 lo = *reinterpret_cast<const uint4*>(K8 + qc.k8o[s][0]);
          const uint4 hi = *reinterpret_cast<const uint4*>(K8 + qc.k8o[s][1]);
          ka[kt][s] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
      }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        S[kt] = QF == QF_FP4 ? mfma32x32x64_fp4(ka[kt][s], q8f[s], S[kt]) : mfma32x32x64_fp8(ka[kt][s], q8f[s], S[kt]);
  }
  // ---- per-key scales and mask.  ALIGN: the block lies in one 64-token block
  //      of the call, so its keys share one scale, folded into cq by the caller.
  if (FP8 && !ALIGN) {
    float4 s4[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        s4[kt][rr] = *reinterpret_cast<const float4*>(cb.sk + key_of(kt, 4 * rr, qc.g));
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        S[kt][4 * rr] *= s4[kt][rr].x;
        S[kt][4 * rr + 1] *= s4[kt][rr].y;
        S[kt][4 * rr + 2] *= s4[kt][rr].z;
        S[kt][4 * rr + 3] *= s4[kt][rr].w;
      }
    // every LDS read of the stage (operands, then scales) before the four
    // products, which alternate between the two score tiles
    __builtin_amdgcn_sched_group_barrier(0x100, QF == QF_FP4 ? 12 : 16, 1);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
  }
  if (!full) {
    // valid iff hi - wl < pk <= hi, i.e. (unsigned)(hi - pk) < wl; with ALIGN
    // also k < size, folded into the band: its top becomes min(hi - pb, size - 1)
    // and its length shrinks by as much (never below zero)
    int base = hi - pb, len = wl;
    if (ALIGN) {
      const int top = min(base, size - 1);
      len = max(wl - (base - top), 0);
      base = top;
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if ((unsigned)(base - key_of(kt, r, qc.g)) >= (unsigned)len) S[kt][r] = -INFINITY;
  }
}

// Probabilities exp2(S cq - m) as bf16 operands (registers 8j..8j+7 of a tile
// are keys 32 kt + 16 j + 8 g + 0..7) and the lane's share of their sum, which
// adds the bf16-rounded values (the weights the P V product uses), two per
// instruction, into one partial sum per score tile.
__device__ __forceinline__ float win_probs(const f32x16 (&S)[2], float cq, float m, bf16x8 (&P)[2][2]) {
  float lk[2] = {0.f, 0.f};
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(S[kt][r], cq, -m));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      P[kt][j] = to_bf16x8(p[8 * j], p[8 * j + 1], p[8 * j + 2], p[8 * j + 3], p[8 * j + 4],
                           p[8 * j + 5], p[8 * j + 6], p[8 * j + 7]);
      const uint4 pw = __builtin_bit_cast(uint4, P[kt][j]);
      lk[kt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw.x), ones, lk[kt], false);
      lk[kt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw.y), ones, lk[kt], false);
      lk[kt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw.z), ones, lk[kt], false);
      lk[kt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw.w), ones, lk[kt], false);
    }
  }
  return lk[0] + lk[1];
}

// One key block of a branch: scores from buffer cb, online softmax, O update.
// With spec, the probabilities are first formed against the running maximum
// as it stands, without the block maximum: a lane whose block sum stays at or
// below SPEC_LIMIT has every probability at or below it.  Over nb blocks the
// two lanes of a query then hold l <= nb * 2^33 and |O| <= l * max|v|, so fp32
// holds them while nb * max|v| stays below about 2^94 (about 2^113 when every
// probability is at most 2^RESCALE_SLACK, as after the maximum path).  Only
// if some lane of the wave exceeds it (its
// maximum rose by more than log2(SPEC_LIMIT) - 6, or the lane has seen no key
// yet) are the scores formed again and the block takes the maximum and
// rescale path; after that every lane's probabilities are at most
// 2^RESCALE_SLACK, so one repeat suffices.  Returns whether an attempt was
// made and failed.
template <int QF, bool ALIGN>
__device__ __forceinline__ bool win_block(const WinBuf& cb, const QueryCtx& qc, int hi, int wl, int pb,
                                          int size, float ks, bool full, bool spec, const bf16x8 (&qf)[8],
                                          const i32x8 (&q8f)[2], f32x16 (&O)[4], float& m_run,
                                          float& l_run) {
  const float cq = ALIGN ? qc.cq * ks : qc.cq;
  f32x16 S[2];
  bf16x8 P[2][2];
  float l_blk = 0.f;
  bool redo = true;
  if (spec) {
    win_scores<QF, ALIGN>(cb, qc, hi, wl, pb, size, full, qf, q8f, S);
    l_blk = win_probs(S, cq, m_run, P);
    redo = __ballot(l_blk > SPEC_LIMIT) != 0;
  }
  if (redo) {
    win_scores<QF, ALIGN>(cb, qc, hi, wl, pb, size, full, qf, q8f, S);
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kt][r]);
    mx = max_with_partner(mx) * cq;
    if (__ballot(mx > m_run + RESCALE_SLACK) != 0) {
      const float m_new = mx > m_run + RESCALE_SLACK ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[dt][r] *= alpha;
      m_run = m_new;
    }
    l_blk = win_probs(S, cq, m_run, P);
  }
  l_run += l_blk;
  const bool failed = spec && redo;
  // ---- O^T += V^T P^T   (lane: O^T[32dt + 8(r/4) + 4g + r%4][query ql]); the
  //      V^T operand of (kt, j, dt): features 32 dt + lane%32, keys
  //      32 kt + 16 j + 8 g + 0..7.  Products in the order (kt, j) outer, dt
  //      inner: consecutive products accumulate into different tiles and share
  //      the P operand; every operand is read before the products start.
  const uint8_t* Vb = reinterpret_cast<const uint8_t*>(cb.V);
  bf16x8 vop[16];
#pragma unroll
  for (int idx = 0; idx < 16; ++idx) {
    const int dt = idx & 3, j = (idx >> 2) & 1, kt = idx >> 3;
    const uint8_t* vp = Vb + (32 * kt + 16 * j) * VST;
    vop[idx] = as_bf16x8(win_read_tr(reinterpret_cast<const uint16_t*>(vp + qc.vo[dt][0])),
                         win_read_tr(reinterpret_cast<const uint16_t*>(vp + qc.vo[dt][1])));
  }
#pragma unroll
  for (int idx = 0; idx < 16; ++idx) O[idx & 3] = mfma32x32x16(vop[idx], P[idx >> 3][(idx >> 2) & 1], O[idx & 3]);
  // operands four products ahead of their use, then two reads per product
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  return failed;
}

__device__ __forceinline__ bool more_blocks(int jj, int nb) { return jj + 1 < nb; }

// One windowed branch over its key blocks: online softmax into O (unnormalised)
// with running max m_run and lane-partial sum l_run.
template <int QF, bool SHORTL>
__device__ __forceinline__ void run_branch(const WinArgs& a, const WinBuf& B0, const WinBuf& B1,
                                           const BranchRange& br, const QueryCtx& qc,
                                           const bf16x8 (&qf)[8], const i32x8 (&q8f)[2],
                                           WinLoads<QF, SHORTL>& ld, f32x16 (&O)[4], float& m_run,
                                           float& l_run) {
  // Quantised keys in frames of at least one block: blocks never straddle a
  // frame end or a 64-token block of the call, so each block's keys share one
  // scale (one uniform load instead of the per-key scale reads).  Otherwise
  // blocks are 64 consecutive group positions.
  constexpr bool ALIGN = QF != QF_BF16 && !SHORTL;
  const int L = a.L;
  const KeyMap& km = br.km;
  const float* kscale_all = br.own_k ? a.k_scales2 : a.k_scales;
  const float* kring_scale = br.own_k && a.ks_ring2 ? a.ks_ring2 : a.ks_ring;
  const float* kscale = kscale_all + ((size_t)qc.b * a.H + qc.h) * a.nblk;
  const bool fblk = a.nbf > 0;        // quantisation blocks restart at every frame
  // token of the call at (sub-frame n, row m), and the end row of the block
  // starting there (blocks also end at quantisation-block boundaries)
  auto tok_of = [&](int n, int m) { return (n * km.dil + km.res - km.frame_offset) * L + m; };
  auto blk_end = [&](int n, int m) {
    return ALIGN ? min(m + BK - ((fblk ? m : tok_of(n, m)) & (BK - 1)), L) : m + BK;
  };
  // key scale of the quantisation block holding (sub-frame n, row m)
  auto scale_at = [&](int n, int m) {
    return fblk ? frame_scales(km, kscale_all, kring_scale, qc.b, qc.h, a.H, a.nblk, a.nbf, n) + m / BK
                : kscale + tok_of(n, m) / BK;
  };
  int n0 = br.p_lo / L, m0 = br.p_lo - (br.p_lo / L) * L;
  // current block: end row e0 and (ALIGN) its key scale (tb0 points at it)
  int e0 = blk_end(n0, m0);
  const float* tb0 = ALIGN ? scale_at(n0, m0) : nullptr;
  float ks0 = ALIGN ? *tb0 : 1.f;
  int nb = br.nb;
  if (ALIGN) {
    nb = 0;
    for (int n = n0, m = m0; n * L + m <= br.p_hi; ++nb) {
      const int e = blk_end(n, m);
      if (e >= L) { ++n; m = 0; } else { m = e; }
    }
  }
  // last valid row of the current block (aligned blocks)
  int dmax0 = ALIGN ? min(e0 - m0, br.p_hi - br.p_lo + 1) - 1 : 0;
  if (ALIGN) {
    win_block_addrs_al<QF, SHORTL>(ld, a, br, qc.b, qc.h, qc.wave, n0, m0, dmax0);
    win_issue_al<QF, SHORTL>(ld, B0, qc.wave);
  } else {
    win_block_addrs<QF, SHORTL>(ld, a, br, qc.b, qc.h, qc.wave, br.p_lo, n0, m0);
    win_issue<QF, SHORTL>(ld, B0, qc.wave);
  }
  win_wait_vmem();
  lds_barrier();
  // Windows are cut at the range's last position p_hi: a range may be part of
  // a branch's key range (the keys of the frames before the query's frame),
  // and a block of consecutive positions may then reach past it.  For a whole
  // range p_hi is already the largest window end of the workgroup.
  const int pq = br.pq0 + qc.mq;                         // this lane's query position
  const int hi = min(min(pq + br.fwd, br.p_last), br.p_hi);   // its window's last key position
  const int wl = max(hi - (pq - br.back) + 1, 0);        // and the window's length (0: no key)
  const int full_lo = br.pq0 + qc.mw_hi - br.back;       // blocks inside every window of the wave
  const int full_hi = min(min(br.pq0 + qc.mw_lo + br.fwd, br.p_last), br.p_hi);
  const int need_lo = br.pq0 + qc.mw_lo - br.back;       // keys inside some window of the wave
  const int need_hi = min(min(br.pq0 + qc.mw_hi + br.fwd, br.p_last), br.p_hi);
  // A block is formed against the running maximum alone only if every lane's
  // window began before it (each lane has a key, hence a finite maximum), the
  // wave's previous block did not fail such an attempt, and fewer than
  // SPEC_TRIES attempts failed in this branch: with widely spread scores the
  // maximum keeps rising, and a failed attempt costs most of a block.
  bool spec = false;
  int nfail = 0;
  // Aligned blocks: the number of blocks after the current one that form a
  // run of interior blocks, each full, valid, past the first block inside
  // every window of the wave (so inside them all, with a speculative attempt
  // allowed), and followed by a full, valid block of the same frame.  Such a
  // block steps its load addresses by one block and needs neither the
  // classification nor the mask; the general step sets the count.
  int run = 0;
  for (int jb = 0; jb < nb; jb += 2) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int jj = jb + half;
      if (jj >= nb) break;
      const WinBuf& cb = half ? B1 : B0;
      const WinBuf& nbuf = half ? B0 : B1;
      int pb, size, n1, m1, e1, dmax1 = 0;
      const float* tb1;
      bool more, full, touch;
      if (ALIGN && run > 0) {
        --run;
        pb = n0 * L + m0;
        size = BK;
        n1 = n0;
        m1 = e0;
        e1 = e0 + BK;
        tb1 = tb0 + 1;
        dmax1 = BK - 1;
        more = true;
        full = true;
        touch = true;
        ld.kb += (size_t)BK * a.H * qk_row_bytes(QF);
        ld.vb += (size_t)BK * a.H * WD * 2;
        win_issue_al<QF, SHORTL>(ld, nbuf, qc.wave);
      } else {
        pb = ALIGN ? n0 * L + m0 : br.p_lo + BK * jj;
        size = ALIGN ? e0 - m0 : BK;
        // next block's (sub-frame, offset, end, token block) and its loads;
        // inside a frame an aligned block starts at the current end with the
        // next token block
        n1 = n0;
        m1 = e0;
        tb1 = tb0;
        if (ALIGN) {
          if (e0 < L) {
            e1 = min(e0 + BK, L);
            tb1 = tb0 + 1;
          } else {
            n1 = n0 + 1;
            m1 = 0;
            e1 = blk_end(n1, 0);
            tb1 = more_blocks(jj, nb) ? scale_at(n1, 0) : tb0;
          }
        } else {
          while (m1 >= L) { m1 -= L; ++n1; }
          e1 = m1 + BK;
        }
        more = jj + 1 < nb;
        if (more) {
          if (ALIGN) {
            // a full next block in the same frame is this block's rows 64 on
            dmax1 = min(e1 - m1, br.p_hi - (n1 * L + m1) + 1) - 1;
            if (dmax0 == BK - 1 && dmax1 == BK - 1 && n1 == n0) {
              ld.kb += (size_t)BK * a.H * qk_row_bytes(QF);
              ld.vb += (size_t)BK * a.H * WD * 2;
            } else {
              win_block_addrs_al<QF, SHORTL>(ld, a, br, qc.b, qc.h, qc.wave, n1, m1, dmax1);
            }
            win_issue_al<QF, SHORTL>(ld, nbuf, qc.wave);
            // the run that starts with the next block (pc: its position)
            const int pc = n1 * L + m1;
            if (qc.active && e1 - m1 == BK && dmax1 == BK - 1 && m1 + 2 * BK <= L && pc + 2 * BK - 1 <= br.p_hi &&
                pc > full_lo && pc + BK - 1 <= full_hi)
              run = 1 + min(min(L - m1 - 2 * BK, br.p_hi - pc - (2 * BK - 1)), full_hi - pc - (BK - 1)) / BK;
          } else {
            // inside one frame, unclamped, the next block's rows are this block's
            // rows 64 positions on
            const bool step = !SHORTL && m0 + BK <= L && n1 == n0 && m1 + BK <= L && pb + 2 * BK - 1 <= br.p_hi;
            if (step) {
#pragma unroll
              for (int j = 0; j < WinGeom<QF, SHORTL>::NJ; ++j) ld.src[j] += ld.inc[j];
            } else {
              win_block_addrs<QF, SHORTL>(ld, a, br, qc.b, qc.h, qc.wave, n1 * L + m1, n1, m1);
            }
            win_issue<QF, SHORTL>(ld, nbuf, qc.wave);
          }
        }
        full = size == BK && pb >= full_lo && pb + BK - 1 <= full_hi;
        // a wave whose rows all lie past the frame's end (the last, partial
        // query tile), or whose windows all miss this block, only loads its
        // share of the block and keeps the barriers: a block masked for every
        // lane adds nothing to O, l or the running maximum
        touch = pb + size - 1 >= need_lo && pb <= need_hi;
      }
      const float ks1 = ALIGN && more ? *tb1 : 1.f;
      if (qc.active && touch) {
        const bool failed = win_block<QF, ALIGN>(cb, qc, hi, wl, pb, size, ks0, full, spec && pb > full_lo,
                                                 qf, q8f, O, m_run, l_run);
        nfail += failed;
        spec = !failed && nfail < SPEC_TRIES;
      }
      win_wait_vmem();
      lds_barrier();
      n0 = n1;
      m0 = m1;
      e0 = e1;
      tb0 = tb1;
      ks0 = ks1;
      dmax0 = dmax1;
    }
  }
}

// Workgroups per CU: three with quantised Q/K in block-aligned frames (one
// key scale per block and uniform load bases leave them near 168 VGPRs: a few
// spilled registers, and 6.6% faster (E4M3) and 7% (E2M1) than at two); two
// for bf16 Q/K and for frames shorter than a block (per-key scales, 64-bit
// per-lane addresses).
template <int QF, bool SHORTL>
constexpr int win_wgs_per_cu() { return QF != QF_BF16 && !SHORTL ? 3 : 2; }

// SHARE (hybrid only): the two windowed branches score the same q and k and
// the DSWA dilation exceeds 1, so the query's own frame is computed once.
template <int QF, bool HYBRID, bool SHORTL, bool SHARE>
__global__ __launch_bounds__(256, (win_wgs_per_cu<QF, SHORTL>())) void win_attn_kernel(WinArgs a) {
  using G = WinGeom<QF, SHORTL>;
  constexpr bool FP8 = G::FP8;
  __shared__ __attribute__((aligned(16))) uint8_t Kb0[G::KBYTES], Kb1[G::KBYTES];
  __shared__ __attribute__((aligned(16))) uint16_t Vb0[G::VBYTES / 2], Vb1[G::VBYTES / 2];
  __shared__ __attribute__((aligned(16))) float sk0[G::SCL ? BK : 1], sk1[G::SCL ? BK : 1];
  const WinBuf B0{Kb0, Vb0, sk0};
  const WinBuf B1{Kb1, Vb1, sk1};
  const int lid = xcd_swizzle(blockIdx.x, gridDim.x);
  const int qt = lid % a.QT;
  const int f = (lid / a.QT) % a.F;
  const int bh = lid / (a.QT * a.F);
  QueryCtx qc;
  qc.b = bh / a.H;
  qc.h = bh % a.H;
  const int Lf = min(a.L, a.T - f * a.L);          // tokens of this frame in the call
  const int m0 = qt * BQ;
  if (m0 >= Lf) return;
  const int m_last_wg = min(m0 + BQ, Lf) - 1;

  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  qc.wave = wave;
  qc.ql = lane % 32;
  qc.g = lane / 32;
  const int m_row = m0 + 32 * wave + qc.ql;        // query row in the frame
  const bool q_valid = m_row < Lf;
  qc.mq = q_valid ? m_row : m_last_wg;             // clamped row for positions / loads
  const size_t tq = (size_t)f * a.L + qc.mq;       // token index of the query
  const size_t tok_stride = (size_t)a.H * WD;
  qc.mw_lo = min(m0 + 32 * wave, m_last_wg);       // wave's query rows (clamped)
  qc.active = m0 + 32 * wave < Lf;
  qc.mw_hi = min(m0 + 32 * wave + 31, m_last_wg);
  // score row of this lane's A operand: key pi(ql) of each 32-key tile
  qc.krow = 16 * (qc.ql / 16) + 8 * ((qc.ql / 4) & 1) + 4 * ((qc.ql / 8) & 1) + (qc.ql & 3);
  // E4M3 K operand: row krow (+32 kt, which leaves the swizzle unchanged),
  // bytes 64 s + 32 g + 16 half
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      qc.k8o[s2][hh] = qc.krow * K8ST + 16 * ((4 * s2 + 2 * qc.g + hh) ^ k8_swz(qc.krow));
  // E2M1 K operand: row krow, bytes 32 s + 16 g (one 16-byte unit)
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) qc.k4o[s2] = qc.krow * K4ST + 16 * ((2 * s2 + qc.g) ^ k4_swz(qc.krow));
  // V^T operand of feature tile dt: rows 8 (G16/2) + s16/4 (+4), features
  // 32 dt + 16 (G16 % 2) + 4 (s16 % 4) .. +3 (+32 kt + 16 j rows leave the swizzle unchanged)
  {
    const int G16 = lane / 16, s16 = lane % 16;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = 8 * (G16 / 2) + s16 / 4 + 4 * e;
        const int cb = 2 * (32 * dt + 16 * (G16 % 2) + 4 * (s16 % 4));
        qc.vo[dt][e] = r * VST + 16 * ((cb / 16) ^ v_swz(r)) + (cb & 15);
      }
  }
  const int b = qc.b, h = qc.h, g = qc.g;

  WinLoads<QF, SHORTL> ld;
  win_load_setup<QF, SHORTL>(ld, wave, a.H);

  // ---- Q operand registers (B operand of S^T = K Q^T) of a branch
  bf16x8 qf[8];
  i32x8 q8f[2];
  auto load_q = [&](const void* qsrc, const float* qscales) {
    float qscale = 1.f;
    if (!FP8) {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(qsrc) + ((size_t)b * a.T + tq) * tok_stride +
                           (size_t)h * WD;
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + 16 * s + 8 * g));
    } else {
      constexpr int QROW = qk_row_bytes(QF);
      const uint8_t* qp = reinterpret_cast<const uint8_t*>(qsrc) + (((size_t)b * a.T + tq) * a.H + h) * QROW;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (QF == QF_FP4) {       // step s: features 64 s + 32 g .. +31 = bytes 32 s + 16 g .. +15
          const uint4 lo = *reinterpret_cast<const uint4*>(qp + 32 * s + 16 * g);
          q8f[s] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
        } else {
          const uint4 lo = *reinterpret_cast<const uint4*>(qp + 64 * s + 32 * g);
          const uint4 hi = *reinterpret_cast<const uint4*>(qp + 64 * s + 32 * g + 16);
          q8f[s] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
      }
      qscale = qscales[((size_t)b * a.H + h) * a.nblk + (a.nbf > 0 ? (size_t)f * a.nbf + qc.mq / 64 : tq / 64)];
    }
    // log2(e) / sqrt(d) (x the query's block scale): scores in exp2 units
    qc.cq = 1.4426950408889634f * 0.08838834764831845f * qscale;
  };
  load_q(a.q, a.q_scales);

  const size_t rowoff = ((size_t)b * a.T + tq) * tok_stride + (size_t)h * WD;
  f32x16 O[4];
  float m_run = -1e30f, l_run = 0.f;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) O[dt] = f32x16{};

  float fac;
  if constexpr (SHARE) {
    // ---- SWA and DSWA with the query's own frame shared.  Inside one frame
    // the two branches' positions differ by a constant, so a window of either
    // (causal or centred) holds the same keys of that frame, with the same
    // scores (both branches score the same q and k): those keys are computed
    // once.  With the other frames split off (SWA: the neighbouring frames;
    // DSWA: the neighbouring frames of the residue group), each branch is the
    // softmax over two disjoint key sets, merged exactly from each set's
    // result o and log-sum-exp (log2 units) lse = m + log2(l):
    //   o = (2^{lse1 - M} o1 + 2^{lse2 - M} o2) / (2^{lse1 - M} + 2^{lse2 - M}),
    //   M = max(lse1, lse2).
    // Each part is a run of whole key blocks over a range of positions:
    // before the frame [p_lo, pq0 - 1], the frame [pq0, pq0 + L - 1], after
    // it (centred windows) [pq0 + L, p_hi].
    float* lse_row = a.ylse + ((size_t)b * a.T + tq) * a.H + h;
    float* yp = a.ypart + rowoff;
    // Each part's range is recomputed (a few scalar operations) rather than
    // kept live; each part is its own copy of the branch loop, which keeps the
    // loops free of register spills.
    auto part = [&](int dil, int which) {
      BranchRange r = branch_range(a, dil, f, m0, m_last_wg);
      const int lo = which == 0 ? r.p_lo : which == 1 ? r.pq0 : r.pq0 + a.L;
      const int hi = which == 0 ? r.pq0 - 1 : which == 1 ? r.pq0 + a.L - 1 : r.p_hi;
      r.p_lo = max(r.p_lo, lo);
      r.p_hi = min(r.p_hi, hi);
      if (r.p_hi < r.p_lo) return;
      r.nb = (r.p_hi - r.p_lo + BK) / BK;
      run_branch<QF, SHORTL>(a, B0, B1, r, qc, qf, q8f, ld, O, m_run, l_run);
    };
    // (1) SWA keys of the other frames -> normalised o and lse, parked
    part(1, 0);
    if (a.centered) part(1, 2);
    {
      const float ls = sum_with_partner(l_run);
      const float rl = ls > 0.f ? 1.f / ls : 0.f;
      if (q_valid) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq)
            *reinterpret_cast<float4*>(yp + 32 * dt + 8 * rq + 4 * g) =
                make_float4(rl * O[dt][4 * rq], rl * O[dt][4 * rq + 1], rl * O[dt][4 * rq + 2],
                            rl * O[dt][4 * rq + 3]);
        if (g == 0) *lse_row = ls > 0.f ? m_run + __log2f(ls) : -1e30f;
      }
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) O[dt] = f32x16{};
    m_run = -1e30f;
    l_run = 0.f;
    // (2) the query's own frame, for both branches (never empty: it holds the query)
    part(1, 1);
    // (3) sig(z_swa) o_swa, merged from (1) and (2) in place in the parked row;
    //     (2) stays in registers
    {
      const float lc = sum_with_partner(l_run);
      const float lse_c = m_run + __log2f(lc);
      if (q_valid) {
        const float lse_s = *lse_row;
        const float mx = fmaxf(lse_s, lse_c);
        const float ws = __builtin_amdgcn_exp2f(lse_s - mx), wc = __builtin_amdgcn_exp2f(lse_c - mx);
        const float gs = 1.f / ((1.f + __expf(-a.gates[h])) * (ws + wc));
        const float fs = gs * ws, fc = gs * wc / lc;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            float4* p4 = reinterpret_cast<float4*>(yp + 32 * dt + 8 * rq + 4 * g);
            const float4 o1 = *p4;
            *p4 = make_float4(fs * o1.x + fc * O[dt][4 * rq], fs * o1.y + fc * O[dt][4 * rq + 1],
                              fs * o1.z + fc * O[dt][4 * rq + 2], fs * o1.w + fc * O[dt][4 * rq + 3]);
          }
      }
    }
    // (4) DSWA keys of the group's other frames, continuing from (2)
    part(a.dil, 0);
    if (a.centered) part(a.dil, 2);
    fac = 1.f / (sum_with_partner(l_run)) / (1.f + __expf(-a.gates[a.H + h]));
  } else {
  // ---- first branch: SWA (or the single requested branch)
  const BranchRange b0 = branch_range(a, HYBRID ? 1 : a.dil, f, m0, m_last_wg);
  run_branch<QF, SHORTL>(a, B0, B1, b0, qc, qf, q8f, ld, O, m_run, l_run);
  fac = 1.f / (sum_with_partner(l_run));
  if (HYBRID) {
    fac *= 1.f / (1.f + __expf(-a.gates[h]));
    // park sig(z_swa) o_swa (fp32) in this query's workspace row
    if (q_valid) {
      float* yp = a.ypart + rowoff;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          *reinterpret_cast<float4*>(yp + 32 * dt + 8 * rq + 4 * g) =
              make_float4(fac * O[dt][4 * rq], fac * O[dt][4 * rq + 1], fac * O[dt][4 * rq + 2],
                          fac * O[dt][4 * rq + 3]);
    }
    // ---- second branch: DSWA
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) O[dt] = f32x16{};
    m_run = -1e30f;
    l_run = 0.f;
    BranchRange b1 = branch_range(a, a.dil, f, m0, m_last_wg);
    if (a.q2) {                                      // the branch has its own q, k (RoPE)
      load_q(a.q2, a.q_scales2);
      b1.own_k = true;
    }
    run_branch<QF, SHORTL>(a, B0, B1, b1, qc, qf, q8f, ld, O, m_run, l_run);
    fac = 1.f / (sum_with_partner(l_run)) / (1.f + __expf(-a.gates[a.H + h]));
  }
  }

  // ---- epilogue: (+ parked first branch + gated GDN branch) -> bf16 output row
  if (!q_valid) return;
  if (HYBRID && !a.o_gdn) {
    // the GDN branch runs beside this kernel: leave both windowed branches' sum
    float* yp = a.ypart + rowoff;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        float4* p4 = reinterpret_cast<float4*>(yp + 32 * dt + 8 * rq + 4 * g);
        const float4 y1 = *p4;
        *p4 = make_float4(fac * O[dt][4 * rq] + y1.x, fac * O[dt][4 * rq + 1] + y1.y,
                          fac * O[dt][4 * rq + 2] + y1.z, fac * O[dt][4 * rq + 3] + y1.w);
      }
    return;
  }
  const float gg = HYBRID ? 1.f / (1.f + __expf(-a.gates[2 * a.H + h])) : 0.f;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = 32 * dt + 8 * rq + 4 * g;
      float y0 = fac * O[dt][4 * rq], y1 = fac * O[dt][4 * rq + 1];
      float y2 = fac * O[dt][4 * rq + 2], y3 = fac * O[dt][4 * rq + 3];
      if (HYBRID) {
        const float4 yp = *reinterpret_cast<const float4*>(a.ypart + rowoff + d0);
        const uint2 og = *reinterpret_cast<const uint2*>(a.o_gdn + rowoff + d0);
        y0 += yp.x + gg * bf16_to_f32(og.x & 0xFFFFu);
        y1 += yp.y + gg * bf16_to_f32(og.x >> 16);
        y2 += yp.z + gg * bf16_to_f32(og.y & 0xFFFFu);
        y3 += yp.w + gg * bf16_to_f32(og.y >> 16);
      }
      *reinterpret_cast<uint2*>(a.out + rowoff + d0) = pack_bf16x4(y0, y1, y2, y3);
    }
}

// y = bf16_rne(ypart + sig(z_gdn[h]) o_gdn): 8 elements per thread (two
// 16-byte fp32 loads, one 16-byte bf16 load and store).
__global__ __launch_bounds__(256) void hlta_combine_kernel(const float* __restrict__ ypart,
                                                           const uint16_t* __restrict__ o_gdn,
                                                           const float* __restrict__ gates,
                                                           uint16_t* __restrict__ out, long n8, int H) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const int h = (int)((i / (WD / 8)) % H);
  const float gg = 1.f / (1.f + __expf(-gates[2 * H + h]));
  const float4 a = reinterpret_cast<const float4*>(ypart)[2 * i];
  const float4 b = reinterpret_cast<const float4*>(ypart)[2 * i + 1];
  const uint4 og = reinterpret_cast<const uint4*>(o_gdn)[i];
  const uint2 lo = pack_bf16x4(a.x + gg * bf16_to_f32(og.x & 0xFFFFu), a.y + gg * bf16_to_f32(og.x >> 16),
                               a.z + gg * bf16_to_f32(og.y & 0xFFFFu), a.w + gg * bf16_to_f32(og.y >> 16));
  const uint2 hi = pack_bf16x4(b.x + gg * bf16_to_f32(og.z & 0xFFFFu), b.y + gg * bf16_to_f32(og.z >> 16),
                               b.z + gg * bf16_to_f32(og.w & 0xFFFFu), b.w + gg * bf16_to_f32(og.w >> 16));
  reinterpret_cast<uint4*>(out)[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
}

hipError_t launch_hlta_combine(const float* ypart, const uint16_t* o_gdn, const float* gates,
                               uint16_t* out, int B, int T, int H, hipStream_t stream) {
  const long n8 = (long)B * T * H * WD / 8;
  if (n8 == 0) return hipSuccess;
  const long nb = (n8 + 255) / 256;
  if (nb > 0x7FFFFFFF) return hipErrorInvalidValue;
  hlta_combine_kernel<<<(unsigned)nb, 256, 0, stream>>>(ypart, o_gdn, gates, out, n8, H);
  return hipGetLastError();
}

long window_workgroups(int B, int T, int H, int L) {
  if (L <= 0) return 0;
  return (long)B * H * ((T + L - 1) / L) * ((L + BQ - 1) / BQ);
}

hipError_t launch_window(const WinArgs& args_in, int qf, bool hybrid, hipStream_t stream) {
  WinArgs a = args_in;
  a.QT = (a.L + BQ - 1) / BQ;
  const long nwg = (long)a.B * a.H * a.F * a.QT;
  if (nwg == 0) return hipSuccess;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (hybrid && !a.ypart) return hipErrorInvalidValue;
  if (qf < QF_BF16 || qf > QF_FP4) return hipErrorInvalidValue;
  dim3 grid((unsigned)nwg);
  const bool shortl = a.L < BK;
  // the own frame is shared when both branches score the same q and k
  const bool share = hybrid && a.dil > 1 && !a.q2;
#define KAIROS_WIN_LAUNCH(QQ, HY, SL, SH) win_attn_kernel<QQ, HY, SL, SH><<<grid, 256, 0, stream>>>(a)
#define KAIROS_WIN_SL(QQ, SL)                                                              \
  if (share) KAIROS_WIN_LAUNCH(QQ, true, SL, true);                                        \
  else if (hybrid) KAIROS_WIN_LAUNCH(QQ, true, SL, false);                                 \
  else KAIROS_WIN_LAUNCH(QQ, false, SL, false);
#define KAIROS_WIN_QF(QQ)                                                                  \
  if (shortl) { KAIROS_WIN_SL(QQ, true) } else { KAIROS_WIN_SL(QQ, false) }
  if (qf == QF_FP4) { KAIROS_WIN_QF(QF_FP4) }
  else if (qf == QF_FP8) { KAIROS_WIN_QF(QF_FP8) }
  else { KAIROS_WIN_QF(QF_BF16) }
#undef KAIROS_WIN_QF
#undef KAIROS_WIN_SL
#undef KAIROS_WIN_LAUNCH
  return hipGetLastError();
}

}  // namespace kairos
