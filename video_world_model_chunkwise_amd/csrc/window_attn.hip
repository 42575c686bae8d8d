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
#include "common.hpp"
#include "launch.hpp"

namespace kairos {

constexpr int WD = 128;          // head dimension
constexpr int BQ = 128;          // queries per workgroup
constexpr int BK = 64;           // keys per block
constexpr int KST = WD + 8;      // Ks row stride (bf16 elements)
constexpr int K8ST = WD + 16;    // K8s row stride (bytes)
constexpr int VST = BK + 4;      // Vt row stride (bf16 elements)

template <bool FP8>
struct WinSmem {
  static constexpr int KBYTES = FP8 ? BK * K8ST : BK * KST * 2;
  uint8_t kbuf[2][KBYTES];
  uint16_t Vt[2][WD][VST];
  float sk[2][BK];
};

// Source pointer of the row (key at group position p) for batch b, head h.
struct KeyMap {
  int L, dil, res, R, T;
  long frame_offset;
  __device__ __forceinline__ long token_or_ring(int p, bool& ring) const {
    const int n = p / L;
    const int m = p - n * L;
    const long f = (long)n * dil + res;             // absolute frame
    if (f >= frame_offset) {
      ring = false;
      return (f - frame_offset) * L + m;             // token index in the call
    }
    ring = true;
    return (long)(f % R) * L + m;                    // row index in the ring
  }
};

template <bool FP8>
__device__ __forceinline__ void win_load_block(const WinArgs& a, const KeyMap& km, int b, int h,
                                               int pb, int p_hi, uint4 (&kr)[4], uint4 (&vr)[4],
                                               float& skr) {
  const int tid = threadIdx.x;
  const size_t tok_stride = (size_t)a.H * WD;
  // V (and bf16 K): 4 consecutive keys x 8 features per thread
  const int kq = tid / 16, dg = tid % 16;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = pb + 4 * kq + j;
    vr[j] = make_uint4(0, 0, 0, 0);
    if (!FP8) kr[j] = make_uint4(0, 0, 0, 0);
    if (p <= p_hi) {
      bool ring;
      const long row = km.token_or_ring(p, ring);
      const size_t off = ring ? (((size_t)b * a.R * a.L + row) * a.H + h) * WD + 8 * dg
                              : ((size_t)b * a.T + row) * tok_stride + (size_t)h * WD + 8 * dg;
      const uint16_t* vsrc = ring ? a.v_ring : a.v;
      vr[j] = *reinterpret_cast<const uint4*>(vsrc + off);
      if (!FP8) {
        const uint16_t* ksrc = ring ? a.k_ring : reinterpret_cast<const uint16_t*>(a.k);
        kr[j] = *reinterpret_cast<const uint4*>(ksrc + off);
      }
    }
  }
  if (FP8) {
    // K codes: key tid / 4, 32 bytes at feature 32 * (tid % 4); FP8 calls have no ring
    const int key = tid / 4, part = tid % 4;
    const int p = pb + key;
    kr[0] = kr[1] = make_uint4(0, 0, 0, 0);
    skr = 0.f;
    if (p <= p_hi) {
      bool ring;
      const long row = km.token_or_ring(p, ring);
      const uint8_t* src = reinterpret_cast<const uint8_t*>(a.k) +
                           ((size_t)b * a.T + row) * tok_stride + (size_t)h * WD + 32 * part;
      kr[0] = *reinterpret_cast<const uint4*>(src);
      kr[1] = *reinterpret_cast<const uint4*>(src + 16);
      if (part == 0) skr = a.k_scales[((size_t)b * a.H + h) * a.nblk + row / 64];
    }
  }
}

__device__ __forceinline__ uint32_t lo16w(uint32_t x) { return x & 0xFFFFu; }
__device__ __forceinline__ uint32_t hi16w(uint32_t x) { return x >> 16; }

template <bool FP8>
__device__ __forceinline__ void win_store_block(WinSmem<FP8>& sm, int buf, const uint4 (&kr)[4],
                                                const uint4 (&vr)[4], float skr) {
  const int tid = threadIdx.x;
  const int kq = tid / 16, dg = tid % 16;
  if (!FP8) {
    uint16_t* Ks = reinterpret_cast<uint16_t*>(sm.kbuf[buf]);
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(Ks + (4 * kq + j) * KST + 8 * dg) = kr[j];
  } else {
    const int key = tid / 4, part = tid % 4;
    uint8_t* K8 = sm.kbuf[buf];
    *reinterpret_cast<uint4*>(K8 + key * K8ST + 32 * part) = kr[0];
    *reinterpret_cast<uint4*>(K8 + key * K8ST + 32 * part + 16) = kr[1];
    if (part == 0) sm.sk[buf][key] = skr;
  }
  const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vr[0]);
  const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vr[1]);
  const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vr[2]);
  const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vr[3]);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    *reinterpret_cast<uint2*>(&sm.Vt[buf][8 * dg + 2 * e][4 * kq]) =
        make_uint2(lo16w(w0[e]) | (lo16w(w1[e]) << 16), lo16w(w2[e]) | (lo16w(w3[e]) << 16));
    *reinterpret_cast<uint2*>(&sm.Vt[buf][8 * dg + 2 * e + 1][4 * kq]) =
        make_uint2(hi16w(w0[e]) | (hi16w(w1[e]) << 16), hi16w(w2[e]) | (hi16w(w3[e]) << 16));
  }
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
  r.km.T = a.T;
  r.km.frame_offset = a.frame_offset;
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

template <bool FP8, bool HYBRID>
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
  // log2(e) / sqrt(d): scores in exp2 units
  const float sc = 1.4426950408889634f * 0.08838834764831845f * qscale;

  const int nbr = HYBRID ? 2 : 1;
  BranchRange br[2];
  br[0] = branch_range(a, HYBRID ? 1 : a.dil, f, m0, m_last_wg);
  if (HYBRID) br[1] = branch_range(a, a.dil, f, m0, m_last_wg);
  const int nb_total = br[0].nb + (HYBRID ? br[1].nb : 0);

  f32x16 O[4];
  f32x16 Y[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    O[dt] = f32x16{};
    Y[dt] = f32x16{};
  }
  float m_run = -1e30f, l_run = 0.f;

  uint4 kr[4], vr[4];
  float skr = 0.f;
  win_load_block<FP8>(a, br[0].km, b, h, br[0].p_lo, br[0].p_hi, kr, vr, skr);
  win_store_block<FP8>(sm, 0, kr, vr, skr);
  __syncthreads();

  int cur_br = 0, jb_in = 0;
  for (int jb = 0; jb < nb_total; ++jb) {
    const int buf = jb & 1;
    // next block's coordinates
    int nbr_i = cur_br, njb = jb_in + 1;
    if (njb >= br[cur_br].nb) { nbr_i = cur_br + 1; njb = 0; }
    const bool has_next = jb + 1 < nb_total;
    if (has_next) {
      const BranchRange& nb_r = br[nbr_i];
      win_load_block<FP8>(a, nb_r.km, b, h, nb_r.p_lo + BK * njb, nb_r.p_hi, kr, vr, skr);
    }

    const BranchRange& cb = br[cur_br];
    const int pb = cb.p_lo + BK * jb_in;
    const int pq = cb.pq0 + mq;                      // this lane's query position
    const bool full = (pb > cb.pq0 + mw_hi - a.w) && (pb + BK - 1 <= cb.pq0 + mw_lo);

    // ---- scores S^T (two 32-key tiles), lane: query ql, keys 32kt + 8(r/4) + 4g + r%4
    f32x16 S[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      S[kt] = f32x16{};
      if (!FP8) {
        const uint16_t* Ks = reinterpret_cast<const uint16_t*>(sm.kbuf[buf]) + (32 * kt + ql) * KST;
#pragma unroll
        for (int s = 0; s < 8; ++s)
          S[kt] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(Ks + 16 * s + 8 * g)), qf[s], S[kt]);
      } else {
        const uint8_t* K8 = sm.kbuf[buf] + (32 * kt + ql) * K8ST;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          uint4 lo = *reinterpret_cast<const uint4*>(K8 + 64 * s + 32 * g);
          uint4 hi = *reinterpret_cast<const uint4*>(K8 + 64 * s + 32 * g + 16);
          i32x8 ka = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          S[kt] = mfma32x32x64_fp8(ka, q8f[s], S[kt]);
        }
      }
    }
    // ---- scale, mask, running max
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kt + 8 * (r / 4) + 4 * g + (r % 4);
        float x = S[kt][r] * sc;
        if (FP8) x *= sm.sk[buf][key];
        if (!full) {
          const int pk = pb + key;
          if (pk > pq || pk <= pq - a.w) x = -INFINITY;
        }
        S[kt][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    if (__ballot(m_new > m_run) != 0) {
      const float alpha = exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[dt][r] *= alpha;
      m_run = m_new;
    }
    // ---- probabilities -> bf16 operands
    bf16x8 P[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = exp2f(S[kt][r] - m_run);
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
        for (int j = 0; j < 2; ++j) {
          uint2 lo = *reinterpret_cast<const uint2*>(vrow + 32 * kt + 16 * j + 4 * g);
          uint2 hi = *reinterpret_cast<const uint2*>(vrow + 32 * kt + 16 * j + 8 + 4 * g);
          O[dt] = mfma32x32x16(as_bf16x8(lo, hi), P[kt][j], O[dt]);
        }
    }

    // ---- end of a branch: normalise and fold into the output accumulator
    if (jb_in + 1 == cb.nb) {
      const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
      const float inv = 1.f / l_tot;
      float gsc = 1.f;
      if (HYBRID) gsc = 1.f / (1.f + __expf(-a.gates[cur_br * a.H + h]));
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

    if (has_next) win_store_block<FP8>(sm, buf ^ 1, kr, vr, skr);
    __syncthreads();
    cur_br = nbr_i;
    jb_in = njb;
  }
  (void)nbr;

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
  if (fp8) {
    if (hybrid) win_attn_kernel<true, true><<<grid, 256, 0, stream>>>(a);
    else win_attn_kernel<true, false><<<grid, 256, 0, stream>>>(a);
  } else {
    if (hybrid) win_attn_kernel<false, true><<<grid, 256, 0, stream>>>(a);
    else win_attn_kernel<false, false><<<grid, 256, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace kairos
