// Gated delta rule forward on gfx950.
//
// Operation (Kairos paper, arXiv 2606.16533 HTML v3, Sec. 2.2.1, Eq. 1-6 and
// step 4; canonical decay placement):
//   S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t,
// S in R^{dv x dk} per (batch, head), fp32.
//
// Two kernels:
//  * gdn_f32_kernel   -- fp32 inputs, exact token order, one workgroup per
//                        (b, h), one thread per row of S (rows of S evolve
//                        independently: row_n(S_t) = a_t row_n(S_{t-1})(I - b k k^T)
//                        + b v_{t,n} k^T).
//  * gdn_chunk_kernel -- bf16 inputs.  Chunks of C = 64 tokens; with
//                        g_t = sum_{s<=t in chunk} log a_s and chunk start state S0:
//        A[t,i] = b_t e^{g_t-g_i} k_t.k_i (i < t),  T = (I + A)^{-1}
//        P[t,i] = e^{g_t-g_i} q_t.k_i (i <= t)
//        X = K S0^T,  R = diag(b)(V - diag(e^g) X),  E = T R
//        O = diag(e^g) Q S0^T + P E
//        S  = e^{g_C} S0 + E^T diag(e^{g_C - g}) K
//    (the recurrence unrolled over the chunk; equal up to rounding).  One
//    workgroup owns 16*NW rows of S of one (b, h) and walks the chunks in
//    order; each wave keeps its 16 rows of S in fp32 MFMA accumulators for
//    the whole sequence, and every state-dependent product of a chunk is
//    chained through registers.  The state-independent part (decays, Gram
//    products, the unit-lower-triangular inverse) is computed by the whole
//    workgroup from LDS-staged K and Q.  The next chunk's K, Q, V, a, b are
//    fetched into registers while the current chunk is processed.
#include "common.hpp"
#include "launch.hpp"

namespace kairos {

// ---------------------------------------------------------------- fp32 path

template <int D>
__global__ __launch_bounds__(D) void gdn_f32_kernel(const float* __restrict__ q,
                                                    const float* __restrict__ k,
                                                    const float* __restrict__ v,
                                                    const float* __restrict__ alpha,
                                                    const float* __restrict__ beta,
                                                    const float* state_in, float* __restrict__ out,
                                                    float* state_out, int T, int H) {
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh % H;
  const int n = threadIdx.x;  // row of S (dv index)
  __shared__ float ks[2][D], qs[2][D];
  float S[D];
  if (state_in) {
    const float4* src = reinterpret_cast<const float4*>(state_in + ((size_t)bh * D + n) * D);
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      float4 x = src[i];
      S[4 * i] = x.x; S[4 * i + 1] = x.y; S[4 * i + 2] = x.z; S[4 * i + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < D; ++i) S[i] = 0.f;
  }
  const size_t tok_stride = (size_t)H * D;
  const float* kp = k + ((size_t)b * T * H + h) * D;
  const float* qp = q + ((size_t)b * T * H + h) * D;
  const float* vp = v + ((size_t)b * T * H + h) * D;
  const float* ap = alpha + (size_t)b * T * H + h;
  const float* bp = beta + (size_t)b * T * H + h;
  float* op = out + ((size_t)b * T * H + h) * D;
  if (T > 0) {
    ks[0][n] = kp[n];
    qs[0][n] = qp[n];
  }
  for (int t = 0; t < T; ++t) {
    const int cur = t & 1;
    // fetch token t+1 while token t is processed
    float kn = 0.f, qn = 0.f;
    if (t + 1 < T) {
      kn = kp[(size_t)(t + 1) * tok_stride + n];
      qn = qp[(size_t)(t + 1) * tok_stride + n];
    }
    const float at = ap[(size_t)t * H], bt = bp[(size_t)t * H];
    const float vt = vp[(size_t)t * tok_stride + n];
    __syncthreads();
    float sk0 = 0.f, sk1 = 0.f;
#pragma unroll
    for (int i = 0; i < D; i += 2) {
      sk0 = fmaf(S[i], ks[cur][i], sk0);
      sk1 = fmaf(S[i + 1], ks[cur][i + 1], sk1);
    }
    const float sk = sk0 + sk1;
    // S <- a (S - b (S k) k^T) + b v k^T  (this row)
    const float c1 = bt * sk, c2 = bt * vt;
    float o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int i = 0; i < D; i += 2) {
      S[i] = fmaf(at, fmaf(-c1, ks[cur][i], S[i]), c2 * ks[cur][i]);
      S[i + 1] = fmaf(at, fmaf(-c1, ks[cur][i + 1], S[i + 1]), c2 * ks[cur][i + 1]);
      o0 = fmaf(S[i], qs[cur][i], o0);
      o1 = fmaf(S[i + 1], qs[cur][i + 1], o1);
    }
    op[(size_t)t * tok_stride + n] = o0 + o1;
    if (t + 1 < T) {
      ks[cur ^ 1][n] = kn;
      qs[cur ^ 1][n] = qn;
    }
  }
  if (state_out) {
    float4* dst = reinterpret_cast<float4*>(state_out + ((size_t)bh * D + n) * D);
#pragma unroll
    for (int i = 0; i < D / 4; ++i)
      dst[i] = make_float4(S[4 * i], S[4 * i + 1], S[4 * i + 2], S[4 * i + 3]);
  }
}

// ---------------------------------------------------------------- bf16 chunkwise path

constexpr int CH = 64;          // chunk length
constexpr int KS_PAD = 8;       // row padding (bf16 elements) of token-major tiles
constexpr int TS = CH + 8;      // row stride of 64-wide bf16 tiles (Kt, Vt, Tb, Pb)
constexpr int AS = CH + 4;      // row stride of the fp32 A tile

template <int D, int NW>
struct GdnSmem {
  static constexpr int NR = 16 * NW;          // rows of S owned by the workgroup
  uint16_t Ks[CH][D + KS_PAD];                // K chunk, token-major
  uint16_t Qs[CH][D + KS_PAD];                // Q chunk, token-major
  uint16_t Kt[D][TS];                         // K chunk, feature-major
  uint16_t Vt[NR][TS];                        // V chunk (owned rows), feature-major
  uint16_t Tb[CH][TS];                        // T = (I + A)^{-1}, bf16
  uint16_t Pb[CH][TS];                        // P, bf16
  float Af[CH][AS];                           // A, fp32
  float gam[CH];                              // e^{g_t}
  float bet[CH];                              // b_t
  float wts[CH];                              // e^{g_C - g_t}
  float g2[CH];                               // g_t in log2 units
};

template <int D, int NW>
struct GdnPrefetch {
  static constexpr int NQUADS = (CH / 4) * (D / 8);                 // 4-token x 8-feature quads
  static constexpr int KQ_PASSES = (NQUADS + 64 * NW - 1) / (64 * NW);
  uint4 k[KQ_PASSES][4];
  uint4 q[KQ_PASSES][4];
  uint2 v[4];
  float a, b;
};

template <int D, int NW>
__device__ __forceinline__ void gdn_fetch(GdnPrefetch<D, NW>& pf, const uint16_t* __restrict__ q,
                                          const uint16_t* __restrict__ k,
                                          const uint16_t* __restrict__ v,
                                          const float* __restrict__ alpha,
                                          const float* __restrict__ beta, int b, int h, int T, int H,
                                          int t0, int n_base) {
  const int tid = threadIdx.x;
  constexpr int DG = D / 8;                 // 16-byte groups per token row
  const size_t tok_stride = (size_t)H * D;
  const size_t base = ((size_t)b * T * H + h) * D;
#pragma unroll
  for (int p = 0; p < GdnPrefetch<D, NW>::KQ_PASSES; ++p) {
    const int u = tid + p * 64 * NW;
    const int dg = u % DG, tq = u / DG;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + 4 * tq + j;
      if (u < GdnPrefetch<D, NW>::NQUADS && t < T) {
        const size_t off = base + (size_t)t * tok_stride + 8 * dg;
        pf.k[p][j] = *reinterpret_cast<const uint4*>(k + off);
        pf.q[p][j] = *reinterpret_cast<const uint4*>(q + off);
      } else {
        pf.k[p][j] = make_uint4(0, 0, 0, 0);
        pf.q[p][j] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  {
    const int nq = tid % (4 * NW), tq = tid / (4 * NW);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + 4 * tq + j;
      pf.v[j] = (t < T) ? *reinterpret_cast<const uint2*>(v + base + (size_t)t * tok_stride +
                                                          n_base + 4 * nq)
                        : make_uint2(0, 0);
    }
  }
  if (tid < 64) {
    const int t = t0 + tid;
    if (t < T) {
      pf.a = alpha[((size_t)b * T + t) * H + h];
      pf.b = beta[((size_t)b * T + t) * H + h];
    } else {
      pf.a = 1.f;   // padding tokens: no decay, no write
      pf.b = 0.f;
    }
  }
}

__device__ __forceinline__ uint32_t lo16(uint32_t x) { return x & 0xFFFFu; }
__device__ __forceinline__ uint32_t hi16(uint32_t x) { return x >> 16; }

template <int D, int NW>
__device__ __forceinline__ void gdn_stage(const GdnPrefetch<D, NW>& pf, GdnSmem<D, NW>& sm) {
  const int tid = threadIdx.x;
  constexpr int DG = D / 8;
#pragma unroll
  for (int p = 0; p < GdnPrefetch<D, NW>::KQ_PASSES; ++p) {
    const int u = tid + p * 64 * NW;
    if (u >= GdnPrefetch<D, NW>::NQUADS) break;
    const int dg = u % DG, tq = u / DG;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<uint4*>(&sm.Ks[4 * tq + j][8 * dg]) = pf.k[p][j];
      *reinterpret_cast<uint4*>(&sm.Qs[4 * tq + j][8 * dg]) = pf.q[p][j];
    }
    // transpose the 4 tokens x 8 features block into Kt[d][t..t+3]
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&pf.k[p][0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&pf.k[p][1]);
    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&pf.k[p][2]);
    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&pf.k[p][3]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint2 even = make_uint2(lo16(w0[e]) | (lo16(w1[e]) << 16), lo16(w2[e]) | (lo16(w3[e]) << 16));
      uint2 odd = make_uint2(hi16(w0[e]) | (hi16(w1[e]) << 16), hi16(w2[e]) | (hi16(w3[e]) << 16));
      *reinterpret_cast<uint2*>(&sm.Kt[8 * dg + 2 * e][4 * tq]) = even;
      *reinterpret_cast<uint2*>(&sm.Kt[8 * dg + 2 * e + 1][4 * tq]) = odd;
    }
  }
  {
    const int nq = tid % (4 * NW), tq = tid / (4 * NW);
    const uint32_t a0 = pf.v[0].x, a1 = pf.v[0].y, b0 = pf.v[1].x, b1 = pf.v[1].y;
    const uint32_t c0 = pf.v[2].x, c1 = pf.v[2].y, d0 = pf.v[3].x, d1 = pf.v[3].y;
    *reinterpret_cast<uint2*>(&sm.Vt[4 * nq + 0][4 * tq]) =
        make_uint2(lo16(a0) | (lo16(b0) << 16), lo16(c0) | (lo16(d0) << 16));
    *reinterpret_cast<uint2*>(&sm.Vt[4 * nq + 1][4 * tq]) =
        make_uint2(hi16(a0) | (hi16(b0) << 16), hi16(c0) | (hi16(d0) << 16));
    *reinterpret_cast<uint2*>(&sm.Vt[4 * nq + 2][4 * tq]) =
        make_uint2(lo16(a1) | (lo16(b1) << 16), lo16(c1) | (lo16(d1) << 16));
    *reinterpret_cast<uint2*>(&sm.Vt[4 * nq + 3][4 * tq]) =
        make_uint2(hi16(a1) | (hi16(b1) << 16), hi16(c1) | (hi16(d1) << 16));
  }
}

// Operand of a 16x16x32 product reducing over 32 consecutive indices
// [k0, k0+32) of a bf16 row, in the register-chaining slot order.
__device__ __forceinline__ bf16x8 row_operand_perm(const uint16_t* row, int k0, int g) {
  uint2 lo = *reinterpret_cast<const uint2*>(row + k0 + 4 * g);
  uint2 hi = *reinterpret_cast<const uint2*>(row + k0 + 16 + 4 * g);
  return as_bf16x8(lo, hi);
}

// Operand from the C registers of two vertically adjacent 16x16 tiles.
__device__ __forceinline__ bf16x8 regs_operand(const f32x4& top, const f32x4& bot) {
  return to_bf16x8(top[0], top[1], top[2], top[3], bot[0], bot[1], bot[2], bot[3]);
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void gdn_chunk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* state_in,
    uint16_t* __restrict__ out, float* state_out, int B, int T, int H) {
  constexpr int NR = 16 * NW;
  constexpr int NT = D / NR;          // row tiles per head
  constexpr int DT = D / 16;          // 16-wide feature tiles
  constexpr int DS = D / 32;          // 32-wide feature slabs
  __shared__ GdnSmem<D, NW> sm;

  const int nblocks = gridDim.x;
  const int lid = xcd_swizzle(blockIdx.x, nblocks);
  const int bh = lid / NT, tile = lid % NT;
  if (bh >= B * H) return;
  const int b = bh / H, h = bh % H;
  const int n_base = tile * NR;

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int l16 = lane % 16, g = lane / 16;
  const int n_w = n_base + 16 * wave;     // first S row of this wave

  // ---- state: S^T tiles in C layout, lane holds S[n_w + l16][16 dt + 4 g + r]
  f32x4 S[DT];
  if (state_in) {
    const float* src = state_in + ((size_t)bh * D + n_w + l16) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      float4 x = *reinterpret_cast<const float4*>(src + 16 * dt + 4 * g);
      S[dt] = f32x4{x.x, x.y, x.z, x.w};
    }
  } else {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) S[dt] = zero4();
  }

  // zero the never-written upper blocks of Tb, Pb (and everything else once)
  for (int i = tid; i < CH * TS; i += 64 * NW) {
    (&sm.Tb[0][0])[i] = 0;
    (&sm.Pb[0][0])[i] = 0;
  }

  const int nchunks = (T + CH - 1) / CH;
  GdnPrefetch<D, NW> pf;
  if (nchunks > 0) gdn_fetch<D, NW>(pf, q, k, v, alpha, beta, b, h, T, H, 0, n_base);
  __syncthreads();
  float a_cur = 1.f, b_cur = 0.f;
  if (nchunks > 0) {
    gdn_stage<D, NW>(pf, sm);
    a_cur = pf.a;
    b_cur = pf.b;
  }
  __syncthreads();

  const size_t tok_stride = (size_t)H * D;

  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * CH;
    if (c + 1 < nchunks) gdn_fetch<D, NW>(pf, q, k, v, alpha, beta, b, h, T, H, t0 + CH, n_base);

    // ---- (1) decays: inclusive scan of log2(a) over the chunk (wave 0)
    if (wave == 0) {
      float x = __log2f(a_cur);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      const float gl = __shfl(x, 63, 64);
      sm.g2[lane] = x;
      sm.gam[lane] = exp2f(x);
      sm.wts[lane] = exp2f(gl - x);
      sm.bet[lane] = b_cur;
    }
    __syncthreads();

    // ---- (2) Gram products: A = strictlower(b e^{dg} K K^T) (fp32), P = lower(e^{dg} Q K^T)
    for (int task = wave; task < 20; task += NW) {
      const bool isP = task >= 10;
      int idx = isP ? task - 10 : task;
      int ti = 0;
      while (idx > ti) { idx -= ti + 1; ++ti; }
      const int tj = idx;                              // tj <= ti
      f32x4 acc = zero4();
      const uint16_t* arow = isP ? &sm.Qs[16 * ti + l16][0] : &sm.Ks[16 * ti + l16][0];
      const uint16_t* brow = &sm.Ks[16 * tj + l16][0];
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(arow + 32 * s + 8 * g));
        bf16x8 bb = as_bf16x8(*reinterpret_cast<const uint4*>(brow + 32 * s + 8 * g));
        acc = mfma16x16x32(a, bb, acc);
      }
      const int col = 16 * tj + l16;
      const float gc = sm.g2[col];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * ti + 4 * g + r;
        const float dec = exp2f(sm.g2[row] - gc);
        if (isP) {
          const float val = (col <= row) ? dec * acc[r] : 0.f;
          sm.Pb[row][col] = (uint16_t)(pack_bf16x2(val, 0.f) & 0xFFFFu);
        } else {
          sm.Af[row][col] = (col < row) ? sm.bet[row] * dec * acc[r] : 0.f;
        }
      }
    }
    __syncthreads();

    // ---- (3) diagonal 16x16 blocks of T by forward substitution (wave 0:
    //      lane -> block g, column l16)
    if (wave == 0) {
      const int blk = g, j = l16;
      float x[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const float* arow = &sm.Af[16 * blk + t][16 * blk];
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int i = 0; i + 1 < t; i += 2) {
          s0 = fmaf(arow[i], x[i], s0);
          s1 = fmaf(arow[i + 1], x[i + 1], s1);
        }
        if (t & 1) s0 = fmaf(arow[t - 1], x[t - 1], s0);
        x[t] = ((t == j) ? 1.f : 0.f) - (s0 + s1);
      }
#pragma unroll
      for (int t = 0; t < 16; ++t)
        sm.Tb[16 * blk + t][16 * blk + j] = (uint16_t)(pack_bf16x2(x[t], 0.f) & 0xFFFFu);
    }
    __syncthreads();

    // ---- (4) T_{h1,h0} = -T_{h1,h1} A_{h1,h0} T_{h0,h0} for the two halves
    //      (K = 16 padded to 32: slots 8g + r <-> k = 4g + r, slots 8g+4.. are zero)
    for (int half = wave; half < 2; half += NW) {
      const int h0 = 2 * half, h1 = 2 * half + 1;
      const float* arow = &sm.Af[16 * h1 + l16][16 * h0 + 4 * g];
      bf16x8 a = to_bf16x8(arow[0], arow[1], arow[2], arow[3], 0.f, 0.f, 0.f, 0.f);
      bf16x8 bb;
      {
        const int col = 16 * h0 + l16;
        const int r0 = 16 * h0 + 4 * g;
        uint2 lo = make_uint2(sm.Tb[r0][col] | ((uint32_t)sm.Tb[r0 + 1][col] << 16),
                              sm.Tb[r0 + 2][col] | ((uint32_t)sm.Tb[r0 + 3][col] << 16));
        bb = as_bf16x8(lo, make_uint2(0, 0));
      }
      f32x4 z = mfma16x16x32(a, bb, zero4());
      uint2 tlo = *reinterpret_cast<const uint2*>(&sm.Tb[16 * h1 + l16][16 * h1 + 4 * g]);
      bf16x8 ta = as_bf16x8(tlo, make_uint2(0, 0));
      bf16x8 zb = to_bf16x8(z[0], z[1], z[2], z[3], 0.f, 0.f, 0.f, 0.f);
      f32x4 t10 = mfma16x16x32(ta, zb, zero4());
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sm.Tb[16 * h1 + 4 * g + r][16 * h0 + l16] = (uint16_t)(pack_bf16x2(-t10[r], 0.f) & 0xFFFFu);
    }
    __syncthreads();

    // ---- (5) lower-left 32x32 block: T_LL = -T_H A_HL T_L
    for (int tj = wave; tj < 2; tj += NW) {
      f32x4 z[2];
#pragma unroll
      for (int zi = 0; zi < 2; ++zi) {
        const float* arow = &sm.Af[32 + 16 * zi + l16][8 * g];
        bf16x8 a = to_bf16x8(arow[0], arow[1], arow[2], arow[3], arow[4], arow[5], arow[6], arow[7]);
        const int col = 16 * tj + l16;
        const int r0 = 8 * g;
        uint4 bw = make_uint4(sm.Tb[r0][col] | ((uint32_t)sm.Tb[r0 + 1][col] << 16),
                              sm.Tb[r0 + 2][col] | ((uint32_t)sm.Tb[r0 + 3][col] << 16),
                              sm.Tb[r0 + 4][col] | ((uint32_t)sm.Tb[r0 + 5][col] << 16),
                              sm.Tb[r0 + 6][col] | ((uint32_t)sm.Tb[r0 + 7][col] << 16));
        z[zi] = mfma16x16x32(a, as_bf16x8(bw), zero4());
      }
      const bf16x8 zb = regs_operand(z[0], z[1]);
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
        bf16x8 ta = row_operand_perm(&sm.Tb[32 + 16 * ti + l16][0], 32, g);
        f32x4 tll = mfma16x16x32(ta, zb, zero4());
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sm.Tb[32 + 16 * ti + 4 * g + r][16 * tj + l16] =
              (uint16_t)(pack_bf16x2(-tll[r], 0.f) & 0xFFFFu);
      }
    }
    __syncthreads();

    // ---- (6) state-dependent products for this wave's 16 rows of S
    {
      // S operand (rows n_w + l16, feature slots) for each 32-wide feature slab
      bf16x8 Sop[DS];
#pragma unroll
      for (int s = 0; s < DS; ++s) Sop[s] = regs_operand(S[2 * s], S[2 * s + 1]);

      // X = K S^T  (lane: X[16 tt + 4g + r][n = l16]);  Y^T = S Q^T (lane: Y^T[4g + r][t = 16 tt + l16])
      f32x4 X[4], Y[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        X[tt] = zero4();
        Y[tt] = zero4();
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          X[tt] = mfma16x16x32(row_operand_perm(&sm.Ks[16 * tt + l16][0], 32 * s, g), Sop[s], X[tt]);
          Y[tt] = mfma16x16x32(Sop[s], row_operand_perm(&sm.Qs[16 * tt + l16][0], 32 * s, g), Y[tt]);
        }
      }
      // R = b (V - e^g X)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int t = 16 * tt + 4 * g;
        const uint2 vv = *reinterpret_cast<const uint2*>(&sm.Vt[16 * wave + l16][t]);
        const float vr[4] = {bf16_to_f32(lo16(vv.x)), bf16_to_f32(hi16(vv.x)),
                             bf16_to_f32(lo16(vv.y)), bf16_to_f32(hi16(vv.y))};
#pragma unroll
        for (int r = 0; r < 4; ++r) X[tt][r] = sm.bet[t + r] * (vr[r] - sm.gam[t + r] * X[tt][r]);
      }
      const bf16x8 Rop0 = regs_operand(X[0], X[1]);
      const bf16x8 Rop1 = regs_operand(X[2], X[3]);
      // E = T R  (lane: E[16 tt + 4g + r][n = l16]); T is lower triangular
      f32x4 E[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        E[tt] = mfma16x16x32(row_operand_perm(&sm.Tb[16 * tt + l16][0], 0, g), Rop0, zero4());
        if (tt >= 2)
          E[tt] = mfma16x16x32(row_operand_perm(&sm.Tb[16 * tt + l16][0], 32, g), Rop1, E[tt]);
      }
      const bf16x8 Eop0 = regs_operand(E[0], E[1]);
      const bf16x8 Eop1 = regs_operand(E[2], E[3]);
      // O^T = e^g Y^T + E^T P^T  (lane: O^T[n = 4g + r][t = 16 tt + l16])
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int t = 16 * tt + l16;
        const float gm = sm.gam[t];
        f32x4 o = f32x4{gm * Y[tt][0], gm * Y[tt][1], gm * Y[tt][2], gm * Y[tt][3]};
        o = mfma16x16x32(Eop0, row_operand_perm(&sm.Pb[t][0], 0, g), o);
        if (tt >= 2) o = mfma16x16x32(Eop1, row_operand_perm(&sm.Pb[t][0], 32, g), o);
        const int tok = t0 + t;
        if (tok < T) {
          uint16_t* dst = out + ((size_t)b * T + tok) * tok_stride + (size_t)h * D + n_w + 4 * g;
          *reinterpret_cast<uint2*>(dst) = pack_bf16x4(o[0], o[1], o[2], o[3]);
        }
      }
      // S <- e^{g_C} S + K^T diag(w) E
      const float gC = sm.gam[CH - 1];
      f32x4 WE[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) WE[tt][r] = sm.wts[16 * tt + 4 * g + r] * E[tt][r];
      const bf16x8 WEop0 = regs_operand(WE[0], WE[1]);
      const bf16x8 WEop1 = regs_operand(WE[2], WE[3]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        f32x4 s = f32x4{gC * S[dt][0], gC * S[dt][1], gC * S[dt][2], gC * S[dt][3]};
        s = mfma16x16x32(row_operand_perm(&sm.Kt[16 * dt + l16][0], 0, g), WEop0, s);
        s = mfma16x16x32(row_operand_perm(&sm.Kt[16 * dt + l16][0], 32, g), WEop1, s);
        S[dt] = s;
      }
    }
    __syncthreads();
    if (c + 1 < nchunks) {
      gdn_stage<D, NW>(pf, sm);
      a_cur = pf.a;
      b_cur = pf.b;
    }
    __syncthreads();
  }

  if (state_out) {
    float* dst = state_out + ((size_t)bh * D + n_w + l16) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(dst + 16 * dt + 4 * g) = make_float4(S[dt][0], S[dt][1], S[dt][2], S[dt][3]);
  }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_gdn_f32(const float* q, const float* k, const float* v, const float* alpha,
                          const float* beta, const float* state_in, float* out, float* state_out,
                          int B, int T, int H, int D, hipStream_t stream) {
  dim3 grid(B * H);
  switch (D) {
    case 32: gdn_f32_kernel<32><<<grid, 32, 0, stream>>>(q, k, v, alpha, beta, state_in, out, state_out, T, H); break;
    case 64: gdn_f32_kernel<64><<<grid, 64, 0, stream>>>(q, k, v, alpha, beta, state_in, out, state_out, T, H); break;
    case 128: gdn_f32_kernel<128><<<grid, 128, 0, stream>>>(q, k, v, alpha, beta, state_in, out, state_out, T, H); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// rows of S per workgroup: fewer rows per workgroup when there are few heads,
// so that the chip has enough independent sequential scans to run.
int gdn_chunk_waves(int B, int H, int D) {
  const long heads = (long)B * H;
  if (D == 64) return heads * 1 >= 192 ? 4 : 2;
  return heads * 2 >= 160 ? 4 : 2;
}

template <int D, int NW>
static hipError_t launch_chunk(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const float* alpha, const float* beta, const float* state_in,
                               uint16_t* out, float* state_out, int B, int T, int H,
                               hipStream_t stream) {
  constexpr int NT = D / (16 * NW);
  int nblk = B * H * NT;
  gdn_chunk_kernel<D, NW><<<nblk, 64 * NW, 0, stream>>>(q, k, v, alpha, beta, state_in, out,
                                                        state_out, B, T, H);
  return hipGetLastError();
}

hipError_t launch_gdn_chunk(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const float* alpha, const float* beta, const float* state_in,
                            uint16_t* out, float* state_out, int B, int T, int H, int D, int nw,
                            hipStream_t stream) {
  if (nw <= 0) nw = gdn_chunk_waves(B, H, D);
  if (D == 128) {
    if (nw == 4) return launch_chunk<128, 4>(q, k, v, alpha, beta, state_in, out, state_out, B, T, H, stream);
    if (nw == 2) return launch_chunk<128, 2>(q, k, v, alpha, beta, state_in, out, state_out, B, T, H, stream);
    if (nw == 8) return launch_chunk<128, 8>(q, k, v, alpha, beta, state_in, out, state_out, B, T, H, stream);
  } else if (D == 64) {
    if (nw == 4) return launch_chunk<64, 4>(q, k, v, alpha, beta, state_in, out, state_out, B, T, H, stream);
    if (nw == 2) return launch_chunk<64, 2>(q, k, v, alpha, beta, state_in, out, state_out, B, T, H, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace kairos
