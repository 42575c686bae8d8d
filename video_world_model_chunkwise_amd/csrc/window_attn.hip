// Causal sliding-window (SWA) and dilated sliding-window (DSWA) softmax
// attention on gfx950, with the fused per-head sigmoid branch-gate epilogue of
// the hybrid layer.
//
// Operation (Kairos paper, arXiv 2606.16533 HTML v3, Sec. 2.2.2):
//   SWA (Eq. 7, causal reading):  o_i = sum_{i-w < j <= i} softmax_j(q_i.k_j / sqrt(d)) v_j
//   DSWA (Eq. 8): SWA over the sequence rearranged so that frames with equal
//   (absolute frame index mod dilation) are contiguous.  Nothing is moved in
//   memory: with f the absolute frame of a token, its group is f mod dil and
//   its position inside the group's sequence is p = (f / dil) * L + offset;
//   keys of query i are the tokens of its group with p_i - w < p_j <= p_i.
//   SWA is the same map with dil = 1, so one code path serves both.
//   Hybrid epilogue: y = sig(z_swa) o_swa + sig(z_dswa) o_dswa + sig(z_gdn) o_gdn.
//
// Work decomposition: one workgroup (4 waves) per (batch, head, frame,
// 128-query tile); query tiles never straddle a frame, so each tile has one
// contiguous key range per branch in group-position space.  Keys are walked
// in blocks of 64 positions; each block's K and V rows are gathered (rows of
// one block may come from two frames, or from the ring of a streamed
// rollout) into double-buffered LDS, K token-major and V feature-major.
// Each wave owns 32 queries: S^T = K Q^T on 32x32 matrix-core tiles with Q
// held in registers, an online softmax in exp2 form (one query per lane, the
// row reduction is within the lane plus one exchange with lane ^ 32), then
// O^T += V^T P^T with P taken straight from the score registers.  With FP8
// Q/K the score product uses the 32x32x64 E4M3 instruction and the per-64-
// token-block scales multiply the fp32 scores; P V stays bf16.
//
// Key order inside a 32-key tile: the score tile's row r maps to key
// pi(r) = 16 j + 8 g + 4 h + i for r = 16 j + 8 h + 4 g + i (bits g and h
// swapped).  With that order the 8 score registers a lane feeds into one
// P V product step are 8 consecutive keys, so each V^T operand is a single
// 16-byte LDS read.
//
// The running maximum is only raised when a block's maximum exceeds it by
// more than 8 (log2 units): probabilities then stay <= 2^8, which is exact
// to rescale away at the end, and the O rescale is skipped in almost every
// block.
//
// Two workgroups share a CU (two waves per SIMD), so one wave's softmax
// arithmetic overlaps the other's matrix products.  To fit, the hybrid
// kernel parks the finished first branch (gated, normalised, fp32) in a
// workspace row per query and adds it back in the epilogue.
#include "common.hpp"
#include "launch.hpp"

namespace kairos {

constexpr int WD = 128;          // head dimension
constexpr int BQ = 128;          // queries per workgroup
constexpr int BK = 64;           // keys per block
constexpr int KST = WD + 8;      // Ks row stride (bf16 elements)
constexpr int K8ST = WD + 16;    // K8s row stride (bytes)
constexpr int VST = BK + 8;      // Vt row stride (bf16 elements)
constexpr float RESCALE_SLACK = 8.f;

template <bool FP8>
struct WinSmem {
  static constexpr int KBYTES = FP8 ? BK * K8ST : BK * KST * 2;
  uint8_t kbuf[2][KBYTES];
  uint16_t Vt[2][WD][VST];
  float sk[2][BK];
};

// Position -> source row map of one branch for one workgroup.
struct KeyMap {
  int L, dil, res, R, frame_offset;
};

// First element of the frame at sub-frame index n of the group: a frame of
// the call, or (frames before the call) a ring slot.
__device__ __forceinline__ const uint8_t* frame_base(const KeyMap& km, const uint8_t* x,
                                                     const uint8_t* ring, int esz, int b, int h,
                                                     int T, int H, int n) {
  const int f = n * km.dil + km.res;                       // absolute frame
  if (f >= km.frame_offset)
    return x + (((size_t)b * T + (size_t)(f - km.frame_offset) * km.L) * H + h) * (size_t)WD * esz;
  return ring + (((size_t)b * km.R + f % km.R) * km.L * (size_t)H + h) * (size_t)WD * esz;
}

// Rows of one 64-key block starting at group position pb (offset m0 in
// sub-frame n0).  For L >= 64 the block spans at most two frames: offsets
// m < L come from frame n0, the rest from frame n0 + 1.  Positions past
// p_hi are clamped to p_hi (masked out of the softmax; clamping keeps loads
// in bounds and loaded values finite).
template <bool SHORTL>
struct BlockRows {
  const uint8_t* b0;
  const uint8_t* b1;
  int pb, m0, n0, p_hi, L;
  size_t rs;                  // bytes between consecutive rows of a frame
  __device__ __forceinline__ const uint8_t* row(const KeyMap& km, const uint8_t* x,
                                                const uint8_t* ring, int esz, int b, int h, int T,
                                                int H, int off) const {
    const int d = min(pb + off, p_hi) - pb;
    const int m = m0 + d;
    if (!SHORTL) {
      const bool second = m >= L;
      return (second ? b1 : b0) + (size_t)(unsigned)(second ? m - L : m) * rs;
    }
    const int n = n0 + m / L;
    return frame_base(km, x, ring, esz, b, h, T, H, n) + (size_t)(m - (m / L) * L) * rs;
  }
  // token (in the call) of the key at block offset off; blocks without ring rows only
  __device__ __forceinline__ int token(const KeyMap& km, int off) const {
    const int d = min(pb + off, p_hi) - pb;
    const int m = m0 + d;
    const int n = n0 + m / L;
    return (n * km.dil + km.res - km.frame_offset) * L + (m - (m / L) * L);
  }
};

template <bool SHORTL>
__device__ __forceinline__ BlockRows<SHORTL> block_rows(const KeyMap& km, const uint8_t* x,
                                                        const uint8_t* ring, int esz, int b, int h,
                                                        int T, int H, int pb, int n0, int m0,
                                                        int p_hi) {
  BlockRows<SHORTL> r;
  r.pb = pb;
  r.m0 = m0;
  r.n0 = n0;
  r.p_hi = p_hi;
  r.L = km.L;
  r.rs = (size_t)H * WD * esz;
  if (!SHORTL) {
    r.b0 = frame_base(km, x, ring, esz, b, h, T, H, n0);
    const int n1 = min(n0 + 1, p_hi / km.L);           // only dereferenced for positions <= p_hi
    r.b1 = frame_base(km, x, ring, esz, b, h, T, H, n1);
  }
  return r;
}

// Global loads of one 64-key block into registers.
//  V: thread -> keys 8*(tid%8) .. +7, features 4*(tid/8) .. +3 (8 loads of 8 bytes)
//  bf16 K: thread -> keys 4*(tid/16) .. +3, features 8*(tid%16) .. +7 (4 loads of 16 bytes)
//  E4M3 K: thread -> key tid/4, bytes 32*(tid%4) .. +31 (2 loads of 16 bytes) + its block scale
template <bool FP8>
struct BlockRegs {
  uint2 v[8];
  uint4 k[FP8 ? 2 : 4];
  float sk;
};

template <bool FP8, bool SHORTL>
__device__ __forceinline__ void win_load_block(const WinArgs& a, const KeyMap& km, int b, int h,
                                               int pb, int n0, int m0, int p_hi, BlockRegs<FP8>& r) {
  const int tid = threadIdx.x;
  const uint8_t* vx = reinterpret_cast<const uint8_t*>(a.v);
  const uint8_t* vring = reinterpret_cast<const uint8_t*>(a.v_ring);
  const BlockRows<SHORTL> vr = block_rows<SHORTL>(km, vx, vring, 2, b, h, a.T, a.H, pb, n0, m0, p_hi);
  {
    const int kq8 = tid % 8, dq = tid / 8;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      r.v[j] = *reinterpret_cast<const uint2*>(vr.row(km, vx, vring, 2, b, h, a.T, a.H, 8 * kq8 + j) + 8 * dq);
  }
  const uint8_t* kx = reinterpret_cast<const uint8_t*>(a.k);
  if (!FP8) {
    const uint8_t* kring = reinterpret_cast<const uint8_t*>(a.k_ring);
    const BlockRows<SHORTL> kr = block_rows<SHORTL>(km, kx, kring, 2, b, h, a.T, a.H, pb, n0, m0, p_hi);
    const int kq = tid / 16, dg = tid % 16;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r.k[j] = *reinterpret_cast<const uint4*>(kr.row(km, kx, kring, 2, b, h, a.T, a.H, 4 * kq + j) + 16 * dg);
  } else {
    // E4M3 codes; FP8 calls have no ring, so rows are tokens of the call
    const BlockRows<SHORTL> kr = block_rows<SHORTL>(km, kx, nullptr, 1, b, h, a.T, a.H, pb, n0, m0, p_hi);
    const int key = tid / 4, part = tid % 4;
    const uint8_t* src = kr.row(km, kx, nullptr, 1, b, h, a.T, a.H, key);
    r.k[0] = *reinterpret_cast<const uint4*>(src + 32 * part);
    r.k[1] = *reinterpret_cast<const uint4*>(src + 32 * part + 16);
    r.sk = a.k_scales[((size_t)b * a.H + h) * a.nblk + kr.token(km, key) / 64];
  }
}

__device__ __forceinline__ uint32_t lo16w(uint32_t x) { return x & 0xFFFFu; }
__device__ __forceinline__ uint32_t hi16w(uint32_t x) { return x >> 16; }
// (low half of a, low half of b) and (high half of a, high half of b)
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

template <bool FP8>
__device__ __forceinline__ void win_store_block(WinSmem<FP8>& sm, int buf, const BlockRegs<FP8>& r) {
  const int tid = threadIdx.x;
  if (!FP8) {
    const int kq = tid / 16, dg = tid % 16;
    uint16_t* Ks = reinterpret_cast<uint16_t*>(sm.kbuf[buf]);
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(Ks + (4 * kq + j) * KST + 8 * dg) = r.k[j];
  } else {
    const int key = tid / 4, part = tid % 4;
    uint8_t* K8 = sm.kbuf[buf];
    *reinterpret_cast<uint4*>(K8 + key * K8ST + 32 * part) = r.k[0];
    *reinterpret_cast<uint4*>(K8 + key * K8ST + 32 * part + 16) = r.k[1];
    if (part == 0) sm.sk[buf][key] = r.sk;
  }
  // V^T: feature row 4 dq + e gets keys 8 kq8 .. +7 (one 16-byte write per feature)
  const int kq8 = tid % 8, dq = tid / 8;
  uint4 w[4];
  w[0] = make_uint4(pack_lo(r.v[0].x, r.v[1].x), pack_lo(r.v[2].x, r.v[3].x),
                    pack_lo(r.v[4].x, r.v[5].x), pack_lo(r.v[6].x, r.v[7].x));
  w[1] = make_uint4(pack_hi(r.v[0].x, r.v[1].x), pack_hi(r.v[2].x, r.v[3].x),
                    pack_hi(r.v[4].x, r.v[5].x), pack_hi(r.v[6].x, r.v[7].x));
  w[2] = make_uint4(pack_lo(r.v[0].y, r.v[1].y), pack_lo(r.v[2].y, r.v[3].y),
                    pack_lo(r.v[4].y, r.v[5].y), pack_lo(r.v[6].y, r.v[7].y));
  w[3] = make_uint4(pack_hi(r.v[0].y, r.v[1].y), pack_hi(r.v[2].y, r.v[3].y),
                    pack_hi(r.v[4].y, r.v[5].y), pack_hi(r.v[6].y, r.v[7].y));
#pragma unroll
  for (int e = 0; e < 4; ++e) *reinterpret_cast<uint4*>(&sm.Vt[buf][4 * dq + e][8 * kq8]) = w[e];
}

// Key range of one branch for one query tile, in group-position space.
struct BranchRange {
  KeyMap km;
  int pq0;      // group position of query row m = 0 of the frame
  int p_lo, p_hi, nb;
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
  const int lo = r.pq0 + m_first - a.w + 1;
  r.p_lo = lo > p_avail ? lo : p_avail;
  r.p_hi = r.pq0 + m_last;
  r.nb = (r.p_hi - r.p_lo + BK) / BK;
  return r;
}

// key offset inside a 64-key block of score register r of tile kt (lane group g)
__device__ __forceinline__ constexpr int key_of(int kt, int r, int g) {
  return 32 * kt + 16 * (r / 8) + 8 * g + 4 * ((r / 4) & 1) + (r & 3);
}

// Per-lane query state shared by the branch loops.
struct QueryCtx {
  int b, h, mq, mw_lo, mw_hi, krow, ql, g;
  float cq;
};

// One windowed branch over its key blocks: online softmax into O (unnormalised)
// with running max m_run and lane-partial sum l_run.
template <bool FP8, bool SHORTL>
__device__ __forceinline__ void run_branch(const WinArgs& a, WinSmem<FP8>& sm, const BranchRange& br,
                                           const QueryCtx& qc, const bf16x8 (&qf)[8],
                                           const i32x8 (&q8f)[2], f32x16 (&O)[4], float& m_run,
                                           float& l_run) {
  const int L = a.L;
  int n0 = br.p_lo / L, m0 = br.p_lo - (br.p_lo / L) * L;
  BlockRegs<FP8> regs;
  win_load_block<FP8, SHORTL>(a, br.km, qc.b, qc.h, br.p_lo, n0, m0, br.p_hi, regs);
  win_store_block<FP8>(sm, 0, regs);
  lds_barrier();
  const int pq = br.pq0 + qc.mq;                         // this lane's query position
  for (int jb = 0; jb < br.nb; ++jb) {
    const int buf = jb & 1;
    const int pb = br.p_lo + BK * jb;
    // next block's (sub-frame, offset)
    int n1 = n0, m1 = m0 + BK;
    while (m1 >= L) { m1 -= L; ++n1; }
    const bool has_next = jb + 1 < br.nb;
    if (has_next) win_load_block<FP8, SHORTL>(a, br.km, qc.b, qc.h, pb + BK, n1, m1, br.p_hi, regs);

    const bool full = (pb > br.pq0 + qc.mw_hi - a.w) && (pb + BK - 1 <= br.pq0 + qc.mw_lo);

    // ---- scores S^T (two 32-key tiles), lane: query ql, key key_of(kt, r, g)
    f32x16 S[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      S[kt] = f32x16{};
      if (!FP8) {
        const uint16_t* Ks = reinterpret_cast<const uint16_t*>(sm.kbuf[buf]) + (32 * kt + qc.krow) * KST;
#pragma unroll
        for (int s = 0; s < 8; ++s)
          S[kt] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(Ks + 16 * s + 8 * qc.g)), qf[s], S[kt]);
      } else {
        const uint8_t* K8 = sm.kbuf[buf] + (32 * kt + qc.krow) * K8ST;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const uint4 lo = *reinterpret_cast<const uint4*>(K8 + 64 * s + 32 * qc.g);
          const uint4 hi = *reinterpret_cast<const uint4*>(K8 + 64 * s + 32 * qc.g + 16);
          const i32x8 ka = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          S[kt] = mfma32x32x64_fp8(ka, q8f[s], S[kt]);
        }
      }
    }
    // ---- key scales, mask, block maximum (before the positive factor cq)
    if (FP8) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float4 s4 = *reinterpret_cast<const float4*>(&sm.sk[buf][key_of(kt, 4 * rr, qc.g)]);
          S[kt][4 * rr] *= s4.x;
          S[kt][4 * rr + 1] *= s4.y;
          S[kt][4 * rr + 2] *= s4.z;
          S[kt][4 * rr + 3] *= s4.w;
        }
    }
    if (!full) {
      // valid iff pq - w < pk <= pq, i.e. (unsigned)(pq - pk) < w
      const int base = pq - pb;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if ((unsigned)(base - key_of(kt, r, qc.g)) >= (unsigned)a.w) S[kt][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * qc.cq;
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
    // ---- probabilities -> bf16 operands: registers 8j..8j+7 of a tile are keys
    //      32 kt + 16 j + 8 g + 0..7
    bf16x8 P[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = __builtin_amdgcn_exp2f(fmaf(S[kt][r], qc.cq, -m_run));
        l_run += p[r];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
        P[kt][j] = to_bf16x8(p[8 * j], p[8 * j + 1], p[8 * j + 2], p[8 * j + 3], p[8 * j + 4],
                             p[8 * j + 5], p[8 * j + 6], p[8 * j + 7]);
    }
    // ---- O^T += V^T P^T   (lane: O^T[32dt + 8(r/4) + 4g + r%4][query ql])
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const uint16_t* vrow = &sm.Vt[buf][32 * dt + qc.ql][0];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          O[dt] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(vrow + 32 * kt + 16 * j + 8 * qc.g)),
                               P[kt][j], O[dt]);
    }
    if (has_next) win_store_block<FP8>(sm, buf ^ 1, regs);
    lds_barrier();
    n0 = n1;
    m0 = m1;
  }
}

template <bool FP8, bool HYBRID, bool SHORTL>
__global__ __launch_bounds__(256, 2) void win_attn_kernel(WinArgs a) {
  __shared__ WinSmem<FP8> sm;
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

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  qc.ql = lane % 32;
  qc.g = lane / 32;
  const int m_row = m0 + 32 * wave + qc.ql;        // query row in the frame
  const bool q_valid = m_row < Lf;
  qc.mq = q_valid ? m_row : m_last_wg;             // clamped row for positions / loads
  const size_t tq = (size_t)f * a.L + qc.mq;       // token index of the query
  const size_t tok_stride = (size_t)a.H * WD;
  qc.mw_lo = min(m0 + 32 * wave, m_last_wg);       // wave's query rows (clamped)
  qc.mw_hi = min(m0 + 32 * wave + 31, m_last_wg);
  // score row of this lane's A operand: key pi(ql) of each 32-key tile
  qc.krow = 16 * (qc.ql / 16) + 8 * ((qc.ql / 4) & 1) + 4 * ((qc.ql / 8) & 1) + (qc.ql & 3);
  const int b = qc.b, h = qc.h, g = qc.g;

  // ---- Q operand registers (B operand of S^T = K Q^T)
  bf16x8 qf[8];
  i32x8 q8f[2];
  float qscale = 1.f;
  if (!FP8) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)b * a.T + tq) * tok_stride +
                         (size_t)h * WD;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + 16 * s + 8 * g));
  } else {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(a.q) + ((size_t)b * a.T + tq) * tok_stride +
                        (size_t)h * WD;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint4 lo = *reinterpret_cast<const uint4*>(qp + 64 * s + 32 * g);
      const uint4 hi = *reinterpret_cast<const uint4*>(qp + 64 * s + 32 * g + 16);
      q8f[s] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    qscale = a.q_scales[((size_t)b * a.H + h) * a.nblk + tq / 64];
  }
  // log2(e) / sqrt(d) (x the query's block scale): scores in exp2 units
  qc.cq = 1.4426950408889634f * 0.08838834764831845f * qscale;

  const size_t rowoff = ((size_t)b * a.T + tq) * tok_stride + (size_t)h * WD;
  f32x16 O[4];
  float m_run = -1e30f, l_run = 0.f;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) O[dt] = f32x16{};

  // ---- first branch: SWA (or the single requested branch)
  const BranchRange b0 = branch_range(a, HYBRID ? 1 : a.dil, f, m0, m_last_wg);
  run_branch<FP8, SHORTL>(a, sm, b0, qc, qf, q8f, O, m_run, l_run);
  float fac = 1.f / (l_run + __shfl_xor(l_run, 32, 64));
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
    const BranchRange b1 = branch_range(a, a.dil, f, m0, m_last_wg);
    run_branch<FP8, SHORTL>(a, sm, b1, qc, qf, q8f, O, m_run, l_run);
    fac = 1.f / (l_run + __shfl_xor(l_run, 32, 64)) / (1.f + __expf(-a.gates[a.H + h]));
  }

  // ---- epilogue: (+ parked first branch + gated GDN branch) -> bf16 output row
  if (!q_valid) return;
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
        y0 += yp.x + gg * bf16_to_f32(lo16w(og.x));
        y1 += yp.y + gg * bf16_to_f32(hi16w(og.x));
        y2 += yp.z + gg * bf16_to_f32(lo16w(og.y));
        y3 += yp.w + gg * bf16_to_f32(hi16w(og.y));
      }
      *reinterpret_cast<uint2*>(a.out + rowoff + d0) = pack_bf16x4(y0, y1, y2, y3);
    }
}

hipError_t launch_window(const WinArgs& args_in, bool fp8, bool hybrid, hipStream_t stream) {
  WinArgs a = args_in;
  a.QT = (a.L + BQ - 1) / BQ;
  const long nwg = (long)a.B * a.H * a.F * a.QT;
  if (nwg == 0) return hipSuccess;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (hybrid && !a.ypart) return hipErrorInvalidValue;
  dim3 grid((unsigned)nwg);
  const bool shortl = a.L < BK;
#define KAIROS_WIN_LAUNCH(F8, HY, SL) win_attn_kernel<F8, HY, SL><<<grid, 256, 0, stream>>>(a)
  if (shortl) {
    if (fp8) { if (hybrid) KAIROS_WIN_LAUNCH(true, true, true); else KAIROS_WIN_LAUNCH(true, false, true); }
    else { if (hybrid) KAIROS_WIN_LAUNCH(false, true, true); else KAIROS_WIN_LAUNCH(false, false, true); }
  } else {
    if (fp8) { if (hybrid) KAIROS_WIN_LAUNCH(true, true, false); else KAIROS_WIN_LAUNCH(true, false, false); }
    else { if (hybrid) KAIROS_WIN_LAUNCH(false, true, false); else KAIROS_WIN_LAUNCH(false, false, false); }
  }
#undef KAIROS_WIN_LAUNCH
  return hipGetLastError();
}

}  // namespace kairos
