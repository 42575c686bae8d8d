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

// Element offset of row m of the frame at sub-frame index n of the group:
// a frame of the call, or (frames before the call) a ring slot.
__device__ __forceinline__ const uint8_t* frame_base(const KeyMap& km, const uint8_t* x,
                                                     const uint8_t* ring, int esz, int b, int h,
                                                     int T, int H, int n) {
  const int f = n * km.dil + km.res;                       // absolute frame
  if (f >= km.frame_offset)
    return x + (((size_t)b * T + (size_t)(f - km.frame_offset) * km.L) * H + h) * (size_t)WD * esz;
  return ring + (((size_t)b * km.R + f % km.R) * km.L * (size_t)H + h) * (size_t)WD * esz;
}

// Source rows of the 64 keys of a block starting at group position pb.  For
// L >= 64 a block spans at most two frames: positions with offset m < L come
// from frame n0, the rest from frame n0 + 1.  Positions past p_hi are clamped
// to p_hi (they are masked out of the softmax; clamping keeps loads in bounds
// and the loaded values finite).
template <bool SHORTL>
struct BlockSrc {
  const uint8_t* base0;
  const uint8_t* base1;
  int m0, L, p_hi, pb;
  size_t rstride;             // bytes between consecutive rows of a frame
  const KeyMap* km;
  const uint8_t* x;
  const uint8_t* ring;
  int esz, b, h, T, H;
  int tok0, tok1;             // token index (in the call) of row 0 of frames n0, n0 + 1
  // token of the key at block offset off; only for blocks without ring rows
  __device__ __forceinline__ int token(int off) const {
    const int p = min(pb + off, p_hi);
    if (!SHORTL) {
      const int m = m0 + (p - pb);
      const bool second = m >= L;
      return (second ? tok1 : tok0) + (second ? m - L : m);
    }
    const int n = p / L, m = p - n * L;
    return (n * km->dil + km->res - km->frame_offset) * L + m;
  }
  __device__ __forceinline__ const uint8_t* row(int off) const {
    const int p = min(pb + off, p_hi);
    if (!SHORTL) {
      const int m = m0 + (p - pb);
      const bool second = m >= L;
      const uint8_t* base = second ? base1 : base0;
      return base + (size_t)(unsigned)(second ? m - L : m) * rstride;
    }
    // frames shorter than a block: walk the frames
    const int n = p / L, m = p - n * L;
    return frame_base(*km, x, ring, esz, b, h, T, H, n) + (size_t)m * rstride;
  }
};

template <bool SHORTL>
__device__ __forceinline__ BlockSrc<SHORTL> block_src(const KeyMap& km, const void* x, const void* ring,
                                                      int esz, int b, int h, int T, int H, int pb,
                                                      int p_hi) {
  BlockSrc<SHORTL> s;
  const int n0 = pb / km.L;
  s.m0 = pb - n0 * km.L;
  s.L = km.L;
  s.p_hi = p_hi;
  s.pb = pb;
  s.rstride = (size_t)H * WD * esz;
  s.km = &km;
  s.x = reinterpret_cast<const uint8_t*>(x);
  s.ring = reinterpret_cast<const uint8_t*>(ring);
  s.esz = esz;
  s.b = b;
  s.h = h;
  s.T = T;
  s.H = H;
  s.base0 = frame_base(km, s.x, s.ring, esz, b, h, T, H, n0);
  // the second frame is only dereferenced for positions <= p_hi, which exist
  const int n1 = min(n0 + 1, p_hi / km.L);
  s.base1 = frame_base(km, s.x, s.ring, esz, b, h, T, H, n1);
  s.tok0 = (n0 * km.dil + km.res - km.frame_offset) * km.L;
  s.tok1 = (n1 * km.dil + km.res - km.frame_offset) * km.L;
  return s;
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
                                               int pb, int p_hi, BlockRegs<FP8>& r) {
  const int tid = threadIdx.x;
  {
    const auto vs = block_src<SHORTL>(km, a.v, a.v_ring, 2, b, h, a.T, a.H, pb, p_hi);
    const int kq8 = tid % 8, dq = tid / 8;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      r.v[j] = *reinterpret_cast<const uint2*>(vs.row(8 * kq8 + j) + 8 * dq);
  }
  if (!FP8) {
    const auto ks = block_src<SHORTL>(km, a.k, a.k_ring, 2, b, h, a.T, a.H, pb, p_hi);
    const int kq = tid / 16, dg = tid % 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) r.k[j] = *reinterpret_cast<const uint4*>(ks.row(4 * kq + j) + 16 * dg);
  } else {
    // E4M3 codes; FP8 calls have no ring, so rows are tokens of the call
    const auto ks = block_src<SHORTL>(km, a.k, nullptr, 1, b, h, a.T, a.H, pb, p_hi);
    const int key = tid / 4, part = tid % 4;
    const uint8_t* src = ks.row(key);
    r.k[0] = *reinterpret_cast<const uint4*>(src + 32 * part);
    r.k[1] = *reinterpret_cast<const uint4*>(src + 32 * part + 16);
    r.sk = a.k_scales[((size_t)b * a.H + h) * a.nblk + ks.token(key) / 64];
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
  const long f_abs = a.frame_offset + f;
  r.km.L = a.L;
  r.km.dil = dil;
  r.km.res = (int)(f_abs % dil);
  r.km.R = a.R;
  r.km.frame_offset = (int)a.frame_offset;
  r.pq0 = (int)(f_abs / dil) * a.L;
  const long f_avail = a.frame_offset - a.R > 0 ? a.frame_offset - a.R : 0;
  const long f1 = f_avail + (((r.km.res - f_avail % dil) % dil) + dil) % dil;   // first frame of the group
  const int p_avail = (int)(f1 / dil) * a.L;
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

template <bool FP8, bool HYBRID, bool SHORTL>
__global__ __launch_bounds__(256) void win_attn_kernel(WinArgs a) {
  __shared__ WinSmem<FP8> sm;
  const int lid = xcd_swizzle(blockIdx.x, gridDim.x);
  const int qt = lid % a.QT;
  const int f = (lid / a.QT) % a.F;
  const int bh = lid / (a.QT * a.F);
  const int b = bh / a.H, h = bh % a.H;
  const int Lf = min(a.L, a.T - f * a.L);          // tokens of this frame in the call
  const int m0 = qt * BQ;
  if (m0 >= Lf) return;
  const int m_last_wg = min(m0 + BQ, Lf) - 1;

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int ql = lane % 32, g = lane / 32;
  const int m_row = m0 + 32 * wave + ql;           // query row in the frame
  const bool q_valid = m_row < Lf;
  const int mq = q_valid ? m_row : m_last_wg;      // clamped row for positions / loads
  const long tq = (long)f * a.L + mq;              // token index of the query
  const size_t tok_stride = (size_t)a.H * WD;
  // wave's query rows (clamped) for the block masking decision
  const int mw_lo = min(m0 + 32 * wave, m_last_wg);
  const int mw_hi = min(m0 + 32 * wave + 31, m_last_wg);
  // score row of this lane's A operand: key pi(ql) of each 32-key tile
  const int krow = 16 * (ql / 16) + 8 * ((ql / 4) & 1) + 4 * ((ql / 8) & 1) + (ql & 3);

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
      uint4 lo = *reinterpret_cast<const uint4*>(qp + 64 * s + 32 * g);
      uint4 hi = *reinterpret_cast<const uint4*>(qp + 64 * s + 32 * g + 16);
      q8f[s] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    qscale = a.q_scales[((size_t)b * a.H + h) * a.nblk + tq / 64];
  }
  // log2(e) / sqrt(d) (x the query's block scale): scores in exp2 units
  const float cq = 1.4426950408889634f * 0.08838834764831845f * qscale;

  // branch 0: SWA (or the single requested branch), branch 1: DSWA (hybrid only)
  const BranchRange b0 = branch_range(a, HYBRID ? 1 : a.dil, f, m0, m_last_wg);
  const BranchRange b1 = HYBRID ? branch_range(a, a.dil, f, m0, m_last_wg) : b0;
  const int nb_total = b0.nb + (HYBRID ? b1.nb : 0);

  f32x16 O[4];
  f32x16 Y[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    O[dt] = f32x16{};
    Y[dt] = f32x16{};
  }
  float m_run = -1e30f, l_run = 0.f;

  BlockRegs<FP8> regs;
  win_load_block<FP8, SHORTL>(a, b0.km, b, h, b0.p_lo, b0.p_hi, regs);
  win_store_block<FP8>(sm, 0, regs);
  __syncthreads();

  for (int jb = 0; jb < nb_total; ++jb) {
    const int buf = jb & 1;
    const bool in1 = HYBRID && jb >= b0.nb;          // uniform
    const int jb_in = in1 ? jb - b0.nb : jb;
    const int cb_nb = in1 ? b1.nb : b0.nb;
    const int pb = (in1 ? b1.p_lo : b0.p_lo) + BK * jb_in;
    const int pq0 = in1 ? b1.pq0 : b0.pq0;
    // prefetch the next block (possibly the first block of branch 1)
    const bool has_next = jb + 1 < nb_total;
    if (has_next) {
      const bool n1 = HYBRID && jb + 1 >= b0.nb;
      if (n1) win_load_block<FP8, SHORTL>(a, b1.km, b, h, b1.p_lo + BK * (jb + 1 - b0.nb), b1.p_hi, regs);
      else win_load_block<FP8, SHORTL>(a, b0.km, b, h, b0.p_lo + BK * (jb + 1), b0.p_hi, regs);
    }

    const int pq = pq0 + mq;                         // this lane's query position
    const bool full = (pb > pq0 + mw_hi - a.w) && (pb + BK - 1 <= pq0 + mw_lo);

    // ---- scores S^T (two 32-key tiles), lane: query ql, key key_of(kt, r, g)
    f32x16 S[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      S[kt] = f32x16{};
      if (!FP8) {
        const uint16_t* Ks = reinterpret_cast<const uint16_t*>(sm.kbuf[buf]) + (32 * kt + krow) * KST;
#pragma unroll
        for (int s = 0; s < 8; ++s)
          S[kt] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(Ks + 16 * s + 8 * g)), qf[s], S[kt]);
      } else {
        const uint8_t* K8 = sm.kbuf[buf] + (32 * kt + krow) * K8ST;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          uint4 lo = *reinterpret_cast<const uint4*>(K8 + 64 * s + 32 * g);
          uint4 hi = *reinterpret_cast<const uint4*>(K8 + 64 * s + 32 * g + 16);
          i32x8 ka = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          S[kt] = mfma32x32x64_fp8(ka, q8f[s], S[kt]);
        }
      }
    }
    // ---- key scales, mask, block maximum (unscaled by cq > 0)
    if (FP8) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float4 s4 = *reinterpret_cast<const float4*>(&sm.sk[buf][key_of(kt, 4 * rr, g)]);
          S[kt][4 * rr] *= s4.x;
          S[kt][4 * rr + 1] *= s4.y;
          S[kt][4 * rr + 2] *= s4.z;
          S[kt][4 * rr + 3] *= s4.w;
        }
    }
    if (!full) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int pk = pb + key_of(kt, r, g);
          if (pk > pq || pk <= pq - a.w) S[kt][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * cq;
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
        p[r] = __builtin_amdgcn_exp2f(fmaf(S[kt][r], cq, -m_run));
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
      const uint16_t* vrow = &sm.Vt[buf][32 * dt + ql][0];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          O[dt] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(vrow + 32 * kt + 16 * j + 8 * g)),
                               P[kt][j], O[dt]);
    }

    // ---- end of a branch: normalise and fold into the output accumulator
    if (jb_in + 1 == cb_nb) {
      const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
      const float inv = 1.f / l_tot;
      float gsc = 1.f;
      if (HYBRID) gsc = 1.f / (1.f + __expf(-a.gates[(in1 ? 1 : 0) * a.H + h]));
      const float fac = gsc * inv;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          Y[dt][r] += fac * O[dt][r];
          O[dt][r] = 0.f;
        }
      m_run = -1e30f;
      l_run = 0.f;
    }

    if (has_next) win_store_block<FP8>(sm, buf ^ 1, regs);
    __syncthreads();
  }

  // ---- epilogue: (+ gated GDN branch) -> bf16 output row of this lane's query
  if (!q_valid) return;
  const size_t rowoff = ((size_t)b * a.T + tq) * tok_stride + (size_t)h * WD;
  float gg = 0.f;
  if (HYBRID) gg = 1.f / (1.f + __expf(-a.gates[2 * a.H + h]));
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = 32 * dt + 8 * rq + 4 * g;
      float y0 = Y[dt][4 * rq], y1 = Y[dt][4 * rq + 1], y2 = Y[dt][4 * rq + 2], y3 = Y[dt][4 * rq + 3];
      if (HYBRID) {
        const uint2 og = *reinterpret_cast<const uint2*>(a.o_gdn + rowoff + d0);
        y0 += gg * bf16_to_f32(lo16w(og.x));
        y1 += gg * bf16_to_f32(hi16w(og.x));
        y2 += gg * bf16_to_f32(lo16w(og.y));
        y3 += gg * bf16_to_f32(hi16w(og.y));
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
