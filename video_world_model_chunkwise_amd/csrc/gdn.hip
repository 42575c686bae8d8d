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

__device__ __forceinline__ uint32_t lo16(uint32_t x) { return x & 0xFFFFu; }
__device__ __forceinline__ uint32_t hi16(uint32_t x) { return x >> 16; }
__device__ __forceinline__ uint16_t bf16_bits(float x) { return (uint16_t)(pack_bf16x2(x, 0.f) & 0xFFFFu); }

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

// Lower-triangular 16x16 tile (ti, tj), tj <= ti, of a 64x64 Gram product
// R_ti . C_tj^T over D features (rows of two token-major LDS tiles).
template <int D>
__device__ __forceinline__ f32x4 gram_tile(const uint16_t* rows_a, const uint16_t* rows_b, int stride,
                                           int ti, int tj, int l16, int g) {
  f32x4 acc = zero4();
  const uint16_t* arow = rows_a + (16 * ti + l16) * stride;
  const uint16_t* brow = rows_b + (16 * tj + l16) * stride;
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
    acc = mfma16x16x32(as_bf16x8(*reinterpret_cast<const uint4*>(arow + 32 * s + 8 * g)),
                       as_bf16x8(*reinterpret_cast<const uint4*>(brow + 32 * s + 8 * g)), acc);
  return acc;
}

__device__ __forceinline__ void tri_index(int idx, int& ti, int& tj) {
  ti = 0;
  while (idx > ti) { idx -= ti + 1; ++ti; }
  tj = idx;
}

// ---- prep: per (b, h, chunk), independent of the state
//   g_t = sum_{s<=t} log2 a_s            (written out, fp32)
//   A   = strictlower(b_t 2^{g_t - g_i} k_t.k_i)
//   T   = (I + A)^{-1}                   (written out, bf16, unit lower triangular)
// T by blocks of 16: diagonal blocks by forward substitution, then the two
// 16x16 off-diagonal blocks of each 32x32 half, then the lower-left 32x32
// block T_LL = -T_H A_HL T_L (block inverse of a lower triangular matrix).
template <int D>
struct PrepSmem {
  uint16_t Ks[CH][D + KS_PAD];
  float Af[CH][AS];
  uint16_t Tb[CH][TS];
  float g2[CH];
  float bet[CH];
};

template <int D>
__global__ __launch_bounds__(256) void gdn_prep_kernel(const uint16_t* __restrict__ k,
                                                       const float* __restrict__ alpha,
                                                       const float* __restrict__ beta,
                                                       uint16_t* __restrict__ t_out,
                                                       float* __restrict__ g_out, int T, int H,
                                                       int nchunks) {
  __shared__ PrepSmem<D> sm;
  const int c = blockIdx.x % nchunks;
  const int bh = blockIdx.x / nchunks;
  const int b = bh / H, h = bh % H;
  const int t0 = c * CH;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int l16 = lane % 16, g = lane / 16;
  const size_t tok_stride = (size_t)H * D;
  const size_t base = ((size_t)b * T * H + h) * D;

  for (int i = tid; i < CH * TS; i += 256) (&sm.Tb[0][0])[i] = 0;
  for (int u = tid; u < CH * D / 8; u += 256) {
    const int t = u / (D / 8), dg = u % (D / 8);
    uint4 x = make_uint4(0, 0, 0, 0);
    if (t0 + t < T) x = *reinterpret_cast<const uint4*>(k + base + (size_t)(t0 + t) * tok_stride + 8 * dg);
    *reinterpret_cast<uint4*>(&sm.Ks[t][8 * dg]) = x;
  }
  if (wave == 0) {
    const int t = t0 + lane;
    const float a = t < T ? alpha[((size_t)b * T + t) * H + h] : 1.f;   // padding: no decay,
    const float bb = t < T ? beta[((size_t)b * T + t) * H + h] : 0.f;   // no write
    float x = __log2f(a);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    sm.g2[lane] = x;
    sm.bet[lane] = bb;
  }
  __syncthreads();

  // A = strictlower(b 2^{dg} K K^T), fp32
  for (int task = wave; task < 10; task += 4) {
    int ti, tj;
    tri_index(task, ti, tj);
    const f32x4 acc = gram_tile<D>(&sm.Ks[0][0], &sm.Ks[0][0], D + KS_PAD, ti, tj, l16, g);
    const int col = 16 * tj + l16;
    const float gc = sm.g2[col];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * ti + 4 * g + r;
      sm.Af[row][col] = (col < row) ? sm.bet[row] * __builtin_amdgcn_exp2f(sm.g2[row] - gc) * acc[r] : 0.f;
    }
  }
  __syncthreads();

  // diagonal 16x16 blocks by forward substitution (wave 0: lane -> block g, column l16)
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
    for (int t = 0; t < 16; ++t) sm.Tb[16 * blk + t][16 * blk + j] = bf16_bits(x[t]);
  }
  __syncthreads();

  // T_{h1,h0} = -T_{h1,h1} A_{h1,h0} T_{h0,h0} for the two 32x32 halves
  // (K = 16 padded to 32: slots 8g + r <-> k = 4g + r, slots 8g+4.. are zero)
  if (wave < 2) {
    const int h0 = 2 * wave, h1 = 2 * wave + 1;
    const float* arow = &sm.Af[16 * h1 + l16][16 * h0 + 4 * g];
    const bf16x8 a = to_bf16x8(arow[0], arow[1], arow[2], arow[3], 0.f, 0.f, 0.f, 0.f);
    const int col = 16 * h0 + l16;
    const int r0 = 16 * h0 + 4 * g;
    const uint2 lo = make_uint2(sm.Tb[r0][col] | ((uint32_t)sm.Tb[r0 + 1][col] << 16),
                                sm.Tb[r0 + 2][col] | ((uint32_t)sm.Tb[r0 + 3][col] << 16));
    const f32x4 z = mfma16x16x32(a, as_bf16x8(lo, make_uint2(0, 0)), zero4());
    const uint2 tlo = *reinterpret_cast<const uint2*>(&sm.Tb[16 * h1 + l16][16 * h1 + 4 * g]);
    const f32x4 t10 = mfma16x16x32(as_bf16x8(tlo, make_uint2(0, 0)),
                                   to_bf16x8(z[0], z[1], z[2], z[3], 0.f, 0.f, 0.f, 0.f), zero4());
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.Tb[16 * h1 + 4 * g + r][16 * h0 + l16] = bf16_bits(-t10[r]);
  }
  __syncthreads();

  // lower-left 32x32 block: T_LL = -T_H A_HL T_L (wave tj: column tile tj)
  if (wave < 2) {
    const int tj = wave;
    f32x4 z[2];
#pragma unroll
    for (int zi = 0; zi < 2; ++zi) {
      const float* arow = &sm.Af[32 + 16 * zi + l16][8 * g];
      const bf16x8 a = to_bf16x8(arow[0], arow[1], arow[2], arow[3], arow[4], arow[5], arow[6], arow[7]);
      const int col = 16 * tj + l16;
      const int r0 = 8 * g;
      const uint4 bw = make_uint4(sm.Tb[r0][col] | ((uint32_t)sm.Tb[r0 + 1][col] << 16),
                                  sm.Tb[r0 + 2][col] | ((uint32_t)sm.Tb[r0 + 3][col] << 16),
                                  sm.Tb[r0 + 4][col] | ((uint32_t)sm.Tb[r0 + 5][col] << 16),
                                  sm.Tb[r0 + 6][col] | ((uint32_t)sm.Tb[r0 + 7][col] << 16));
      z[zi] = mfma16x16x32(a, as_bf16x8(bw), zero4());
    }
    const bf16x8 zb = regs_operand(z[0], z[1]);
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      const f32x4 tll = mfma16x16x32(row_operand_perm(&sm.Tb[32 + 16 * ti + l16][0], 32, g), zb, zero4());
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.Tb[32 + 16 * ti + 4 * g + r][16 * tj + l16] = bf16_bits(-tll[r]);
    }
  }
  __syncthreads();

  // write T (64 x 64 bf16, row-major) and g
  uint16_t* tdst = t_out + ((size_t)bh * nchunks + c) * CH * CH;
  for (int u = tid; u < CH * CH / 8; u += 256) {
    const int row = u / 8, cg = u % 8;
    *reinterpret_cast<uint4*>(tdst + row * CH + 8 * cg) = *reinterpret_cast<const uint4*>(&sm.Tb[row][8 * cg]);
  }
  if (wave == 0) g_out[((size_t)bh * nchunks + c) * CH + lane] = sm.g2[lane];
}

// ---- scan: per (b, h, 16*NW rows of S), chunks in order
//
// Staging maps (token quad, feature group) to lanes so that global loads read
// >= 32 contiguous bytes per row while the transposed LDS writes of one
// 32-lane phase land on distinct banks: 4 consecutive lanes share a row,
// 16 rows per wave, and the wave index selects the next feature groups.
__device__ __forceinline__ int kq_dgroup(int u) { return 4 * (u / 64) + (u % 4); }
__device__ __forceinline__ int kq_tquad(int u) { return (u % 64) / 4; }
template <int D, int NW>
struct ScanSmem {
  static constexpr int NR = 16 * NW;
  uint16_t Ks[2][CH][D + KS_PAD];     // K chunk, token-major
  uint16_t Qs[2][CH][D + KS_PAD];     // Q chunk, token-major
  uint16_t Kt[2][D][TS];              // K chunk, feature-major
  uint16_t Vt[2][NR][TS];             // V chunk (owned rows), feature-major
  uint16_t Tb[2][CH][TS];             // T = (I + A)^{-1}
  float g2[2][CH];                    // g_t (log2 units)
  float gam[2][CH];                   // 2^{g_t}
  float wts[2][CH];                   // 2^{g_C - g_t}
  float bet[2][CH];                   // b_t
  uint16_t Pb[CH][TS];                // P = lower(2^{dg} Q K^T)
};

template <int D, int NW>
struct ScanPrefetch {
  static constexpr int NQUADS = (CH / 4) * (D / 8);                 // 4-token x 8-feature quads
  static constexpr int KQ_PASSES = (NQUADS + 64 * NW - 1) / (64 * NW);
  static constexpr int T_UNITS = CH * CH / 8;                       // 16-byte units of T
  static constexpr int T_PASSES = (T_UNITS + 64 * NW - 1) / (64 * NW);
  uint4 k[KQ_PASSES][4];
  uint4 q[KQ_PASSES][4];
  uint2 v[4];
  uint4 t[T_PASSES];
  float g, b;
};

template <int D, int NW>
__device__ __forceinline__ void scan_fetch(ScanPrefetch<D, NW>& pf, const uint16_t* __restrict__ q,
                                           const uint16_t* __restrict__ k,
                                           const uint16_t* __restrict__ v,
                                           const float* __restrict__ beta,
                                           const uint16_t* __restrict__ t_in,
                                           const float* __restrict__ g_in, int b, int h, int bh, int T,
                                           int H, int c, int nchunks, int n_base) {
  // Branch-free: rows past the sequence are clamped to its last token (real,
  // finite data).  They need no zeroing: such tokens get b = 0 when staged, so
  // their rows of R and E are exactly zero and they add nothing to S, and
  // T = (I + A)^{-1} is the identity on them; their outputs are not stored.
  // Without branches the memory counters stay exact, so waits never drain
  // unrelated stores.
  const int tid = threadIdx.x;
  constexpr int DG = D / 8;
  const int t0 = c * CH;
  const size_t tok_stride = (size_t)H * D;
  const size_t base = ((size_t)b * T * H + h) * D;
#pragma unroll
  for (int p = 0; p < ScanPrefetch<D, NW>::KQ_PASSES; ++p) {
    const int u = min(tid + p * 64 * NW, ScanPrefetch<D, NW>::NQUADS - 1);
    const int dg = kq_dgroup(u), tq = kq_tquad(u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = min(t0 + 4 * tq + j, T - 1);
      const size_t off = base + (size_t)t * tok_stride + 8 * dg;
      pf.k[p][j] = *reinterpret_cast<const uint4*>(k + off);
      pf.q[p][j] = *reinterpret_cast<const uint4*>(q + off);
    }
  }
  {
    const int nq = kq_dgroup(tid), tq = kq_tquad(tid);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = min(t0 + 4 * tq + j, T - 1);
      pf.v[j] = *reinterpret_cast<const uint2*>(v + base + (size_t)t * tok_stride + n_base + 4 * nq);
    }
  }
  const uint16_t* tsrc = t_in + ((size_t)bh * nchunks + c) * CH * CH;
#pragma unroll
  for (int p = 0; p < ScanPrefetch<D, NW>::T_PASSES; ++p) {
    const int u = min(tid + p * 64 * NW, ScanPrefetch<D, NW>::T_UNITS - 1);
    pf.t[p] = *reinterpret_cast<const uint4*>(tsrc + 8 * u);
  }
  const int lt = tid % 64;
  pf.g = g_in[((size_t)bh * nchunks + c) * CH + lt];
  pf.b = beta[((size_t)b * T + min(t0 + lt, T - 1)) * H + h];
}

template <int D, int NW>
__device__ __forceinline__ void scan_stage(const ScanPrefetch<D, NW>& pf, ScanSmem<D, NW>& sm, int buf,
                                           int t0, int T) {
  const int tid = threadIdx.x;
  constexpr int DG = D / 8;
#pragma unroll
  for (int p = 0; p < ScanPrefetch<D, NW>::KQ_PASSES; ++p) {
    const int u = tid + p * 64 * NW;
    if (u >= ScanPrefetch<D, NW>::NQUADS) break;
    const int dg = kq_dgroup(u), tq = kq_tquad(u);
    const uint4* kk = pf.k[p];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<uint4*>(&sm.Ks[buf][4 * tq + j][8 * dg]) = pf.k[p][j];
      *reinterpret_cast<uint4*>(&sm.Qs[buf][4 * tq + j][8 * dg]) = pf.q[p][j];
    }
    // transpose the 4 tokens x 8 features block into Kt[d][t..t+3]
    const uint32_t w0[4] = {kk[0].x, kk[0].y, kk[0].z, kk[0].w};
    const uint32_t w1[4] = {kk[1].x, kk[1].y, kk[1].z, kk[1].w};
    const uint32_t w2[4] = {kk[2].x, kk[2].y, kk[2].z, kk[2].w};
    const uint32_t w3[4] = {kk[3].x, kk[3].y, kk[3].z, kk[3].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint2 even = make_uint2(lo16(w0[e]) | (lo16(w1[e]) << 16), lo16(w2[e]) | (lo16(w3[e]) << 16));
      const uint2 odd = make_uint2(hi16(w0[e]) | (hi16(w1[e]) << 16), hi16(w2[e]) | (hi16(w3[e]) << 16));
      *reinterpret_cast<uint2*>(&sm.Kt[buf][8 * dg + 2 * e][4 * tq]) = even;
      *reinterpret_cast<uint2*>(&sm.Kt[buf][8 * dg + 2 * e + 1][4 * tq]) = odd;
    }
  }
  {
    const int nq = kq_dgroup(tid), tq = kq_tquad(tid);
    const uint2* vv = pf.v;
    const uint32_t a0 = vv[0].x, a1 = vv[0].y, b0 = vv[1].x, b1 = vv[1].y;
    const uint32_t c0 = vv[2].x, c1 = vv[2].y, d0 = vv[3].x, d1 = vv[3].y;
    *reinterpret_cast<uint2*>(&sm.Vt[buf][4 * nq + 0][4 * tq]) =
        make_uint2(lo16(a0) | (lo16(b0) << 16), lo16(c0) | (lo16(d0) << 16));
    *reinterpret_cast<uint2*>(&sm.Vt[buf][4 * nq + 1][4 * tq]) =
        make_uint2(hi16(a0) | (hi16(b0) << 16), hi16(c0) | (hi16(d0) << 16));
    *reinterpret_cast<uint2*>(&sm.Vt[buf][4 * nq + 2][4 * tq]) =
        make_uint2(lo16(a1) | (lo16(b1) << 16), lo16(c1) | (lo16(d1) << 16));
    *reinterpret_cast<uint2*>(&sm.Vt[buf][4 * nq + 3][4 * tq]) =
        make_uint2(hi16(a1) | (hi16(b1) << 16), hi16(c1) | (hi16(d1) << 16));
  }
#pragma unroll
  for (int p = 0; p < ScanPrefetch<D, NW>::T_PASSES; ++p) {
    const int u = tid + p * 64 * NW;
    if (u < ScanPrefetch<D, NW>::T_UNITS)
      *reinterpret_cast<uint4*>(&sm.Tb[buf][u / 8][8 * (u % 8)]) = pf.t[p];
  }
  if (tid < 64) {
    const float gl = __shfl(pf.g, 63, 64);
    sm.g2[buf][tid] = pf.g;
    sm.gam[buf][tid] = __builtin_amdgcn_exp2f(pf.g);
    sm.wts[buf][tid] = __builtin_amdgcn_exp2f(gl - pf.g);
    sm.bet[buf][tid] = t0 + tid < T ? pf.b : 0.f;
  }
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void gdn_scan_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ beta, const uint16_t* __restrict__ t_in, const float* __restrict__ g_in,
    const float* state_in, uint16_t* __restrict__ out, float* state_out, int B, int T, int H) {
  constexpr int NR = 16 * NW;
  constexpr int NT = D / NR;          // row tiles per head
  constexpr int DT = D / 16;          // 16-wide feature tiles
  constexpr int DS = D / 32;          // 32-wide feature slabs
  __shared__ ScanSmem<D, NW> sm;

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
      const float4 x = *reinterpret_cast<const float4*>(src + 16 * dt + 4 * g);
      S[dt] = f32x4{x.x, x.y, x.z, x.w};
    }
  } else {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) S[dt] = zero4();
  }
  for (int i = tid; i < CH * TS; i += 64 * NW) (&sm.Pb[0][0])[i] = 0;   // upper blocks stay 0

  const int nchunks = (T + CH - 1) / CH;
  ScanPrefetch<D, NW> pf;
  if (nchunks > 0) {
    scan_fetch<D, NW>(pf, q, k, v, beta, t_in, g_in, b, h, bh, T, H, 0, nchunks, n_base);
    scan_stage<D, NW>(pf, sm, 0, 0, T);
  }
  lds_barrier();

  const size_t tok_stride = (size_t)H * D;
  // outputs of the previous chunk, stored one iteration late so that their
  // completion never sits on a chunk's critical path
  uint2 o_prev0 = make_uint2(0, 0), o_prev1 = o_prev0, o_prev2 = o_prev0, o_prev3 = o_prev0;
  int t0_prev = -1;
  uint16_t* const out_bh = out + (size_t)b * T * tok_stride + (size_t)h * D + n_w + 4 * g;
#define KAIROS_STORE_PREV()                                                              \
  if (t0_prev >= 0) {                                                                    \
    const int tk = t0_prev + l16;                                                        \
    if (tk < T) *reinterpret_cast<uint2*>(out_bh + (size_t)tk * tok_stride) = o_prev0;   \
    if (tk + 16 < T) *reinterpret_cast<uint2*>(out_bh + (size_t)(tk + 16) * tok_stride) = o_prev1; \
    if (tk + 32 < T) *reinterpret_cast<uint2*>(out_bh + (size_t)(tk + 32) * tok_stride) = o_prev2; \
    if (tk + 48 < T) *reinterpret_cast<uint2*>(out_bh + (size_t)(tk + 48) * tok_stride) = o_prev3; \
  }
  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * CH;
    const int cur = c & 1;
    KAIROS_STORE_PREV();
    if (c + 1 < nchunks)
      scan_fetch<D, NW>(pf, q, k, v, beta, t_in, g_in, b, h, bh, T, H, c + 1, nchunks, n_base);

    // ---- P = lower(2^{g_t - g_i} Q K^T)
    // (computed as the tile (tj, ti) of K Q^T: lane holds P[t = 16 ti + l16][i = 16 tj + 4 g + r],
    //  four consecutive entries of a row of P, written as one 8-byte store)
    for (int task = wave; task < 10; task += NW) {
      int ti, tj;
      tri_index(task, ti, tj);
      const f32x4 acc = gram_tile<D>(&sm.Ks[cur][0][0], &sm.Qs[cur][0][0], D + KS_PAD, tj, ti, l16, g);
      const int t = 16 * ti + l16;
      const int i0 = 16 * tj + 4 * g;
      const float gt = sm.g2[cur][t];
      const float4 gi = *reinterpret_cast<const float4*>(&sm.g2[cur][i0]);
      const float p0 = i0 <= t ? __builtin_amdgcn_exp2f(gt - gi.x) * acc[0] : 0.f;
      const float p1 = i0 + 1 <= t ? __builtin_amdgcn_exp2f(gt - gi.y) * acc[1] : 0.f;
      const float p2 = i0 + 2 <= t ? __builtin_amdgcn_exp2f(gt - gi.z) * acc[2] : 0.f;
      const float p3 = i0 + 3 <= t ? __builtin_amdgcn_exp2f(gt - gi.w) * acc[3] : 0.f;
      *reinterpret_cast<uint2*>(&sm.Pb[t][i0]) = pack_bf16x4(p0, p1, p2, p3);
    }
    lds_barrier();

    // ---- state-dependent products for this wave's 16 rows of S
    {
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
          X[tt] = mfma16x16x32(row_operand_perm(&sm.Ks[cur][16 * tt + l16][0], 32 * s, g), Sop[s], X[tt]);
          Y[tt] = mfma16x16x32(Sop[s], row_operand_perm(&sm.Qs[cur][16 * tt + l16][0], 32 * s, g), Y[tt]);
        }
      }
      // R = b (V - 2^g X)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int t = 16 * tt + 4 * g;
        const uint2 vv = *reinterpret_cast<const uint2*>(&sm.Vt[cur][16 * wave + l16][t]);
        const float vr[4] = {bf16_to_f32(lo16(vv.x)), bf16_to_f32(hi16(vv.x)),
                             bf16_to_f32(lo16(vv.y)), bf16_to_f32(hi16(vv.y))};
        const float4 bt = *reinterpret_cast<const float4*>(&sm.bet[cur][t]);
        const float4 gm = *reinterpret_cast<const float4*>(&sm.gam[cur][t]);
        X[tt][0] = bt.x * (vr[0] - gm.x * X[tt][0]);
        X[tt][1] = bt.y * (vr[1] - gm.y * X[tt][1]);
        X[tt][2] = bt.z * (vr[2] - gm.z * X[tt][2]);
        X[tt][3] = bt.w * (vr[3] - gm.w * X[tt][3]);
      }
      const bf16x8 Rop0 = regs_operand(X[0], X[1]);
      const bf16x8 Rop1 = regs_operand(X[2], X[3]);
      // E = T R  (lane: E[16 tt + 4g + r][n = l16]); T is lower triangular
      f32x4 E[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        E[tt] = mfma16x16x32(row_operand_perm(&sm.Tb[cur][16 * tt + l16][0], 0, g), Rop0, zero4());
        if (tt >= 2)
          E[tt] = mfma16x16x32(row_operand_perm(&sm.Tb[cur][16 * tt + l16][0], 32, g), Rop1, E[tt]);
      }
      const bf16x8 Eop0 = regs_operand(E[0], E[1]);
      const bf16x8 Eop1 = regs_operand(E[2], E[3]);
      // O^T = 2^g Y^T + E^T P^T  (lane: O^T[n = 4g + r][t = 16 tt + l16])
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int t = 16 * tt + l16;
        const float gm = sm.gam[cur][t];
        f32x4 o = f32x4{gm * Y[tt][0], gm * Y[tt][1], gm * Y[tt][2], gm * Y[tt][3]};
        o = mfma16x16x32(Eop0, row_operand_perm(&sm.Pb[t][0], 0, g), o);
        if (tt >= 2) o = mfma16x16x32(Eop1, row_operand_perm(&sm.Pb[t][0], 32, g), o);
        const uint2 packed = pack_bf16x4(o[0], o[1], o[2], o[3]);
        if (tt == 0) o_prev0 = packed;
        else if (tt == 1) o_prev1 = packed;
        else if (tt == 2) o_prev2 = packed;
        else o_prev3 = packed;
      }
      t0_prev = t0;
      // S <- 2^{g_C} S + K^T diag(w) E
      const float gC = sm.gam[cur][CH - 1];
      f32x4 WE[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const float4 w4 = *reinterpret_cast<const float4*>(&sm.wts[cur][16 * tt + 4 * g]);
        WE[tt] = f32x4{w4.x * E[tt][0], w4.y * E[tt][1], w4.z * E[tt][2], w4.w * E[tt][3]};
      }
      const bf16x8 WEop0 = regs_operand(WE[0], WE[1]);
      const bf16x8 WEop1 = regs_operand(WE[2], WE[3]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        f32x4 s = f32x4{gC * S[dt][0], gC * S[dt][1], gC * S[dt][2], gC * S[dt][3]};
        s = mfma16x16x32(row_operand_perm(&sm.Kt[cur][16 * dt + l16][0], 0, g), WEop0, s);
        s = mfma16x16x32(row_operand_perm(&sm.Kt[cur][16 * dt + l16][0], 32, g), WEop1, s);
        S[dt] = s;
      }
    }
    if (c + 1 < nchunks) scan_stage<D, NW>(pf, sm, cur ^ 1, t0 + CH, T);
    lds_barrier();
  }
  KAIROS_STORE_PREV();
#undef KAIROS_STORE_PREV

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
  if (D == 64) return heads >= 192 ? 4 : (heads >= 48 ? 2 : 1);
  return heads >= 64 ? 4 : (heads >= 16 ? 2 : 1);
}

size_t gdn_chunk_workspace(int B, int T, int H) {
  const size_t nchunks = (size_t)(T + CH - 1) / CH;
  const size_t tb = (size_t)B * H * nchunks * CH * CH * 2;
  const size_t gb = (size_t)B * H * nchunks * CH * 4;
  return ((tb + 255) / 256) * 256 + gb;
}

template <int D, int NW>
static hipError_t launch_scan(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const float* beta, const uint16_t* t_ws, const float* g_ws,
                              const float* state_in, uint16_t* out, float* state_out, int B, int T,
                              int H, hipStream_t stream) {
  constexpr int NT = D / (16 * NW);
  const int nblk = B * H * NT;
  gdn_scan_kernel<D, NW><<<nblk, 64 * NW, 0, stream>>>(q, k, v, beta, t_ws, g_ws, state_in, out,
                                                       state_out, B, T, H);
  return hipGetLastError();
}

hipError_t launch_gdn_chunk(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const float* alpha, const float* beta, const float* state_in,
                            uint16_t* out, float* state_out, int B, int T, int H, int D, int nw,
                            void* workspace, hipStream_t stream) {
  if (nw <= 0) nw = gdn_chunk_waves(B, H, D);
  const int nchunks = (T + CH - 1) / CH;
  const size_t nt = (size_t)B * H * nchunks;
  uint16_t* t_ws = reinterpret_cast<uint16_t*>(workspace);
  float* g_ws = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) +
                                         ((nt * CH * CH * 2 + 255) / 256) * 256);
  if (nchunks > 0) {
    if (nt > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (D == 128) gdn_prep_kernel<128><<<(unsigned)nt, 256, 0, stream>>>(k, alpha, beta, t_ws, g_ws, T, H, nchunks);
    else if (D == 64) gdn_prep_kernel<64><<<(unsigned)nt, 256, 0, stream>>>(k, alpha, beta, t_ws, g_ws, T, H, nchunks);
    else return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (D == 128) {
    if (nw == 4) return launch_scan<128, 4>(q, k, v, beta, t_ws, g_ws, state_in, out, state_out, B, T, H, stream);
    if (nw == 2) return launch_scan<128, 2>(q, k, v, beta, t_ws, g_ws, state_in, out, state_out, B, T, H, stream);
    if (nw == 1) return launch_scan<128, 1>(q, k, v, beta, t_ws, g_ws, state_in, out, state_out, B, T, H, stream);
  } else if (D == 64) {
    if (nw == 4) return launch_scan<64, 4>(q, k, v, beta, t_ws, g_ws, state_in, out, state_out, B, T, H, stream);
    if (nw == 2) return launch_scan<64, 2>(q, k, v, beta, t_ws, g_ws, state_in, out, state_out, B, T, H, stream);
    if (nw == 1) return launch_scan<64, 1>(q, k, v, beta, t_ws, g_ws, state_in, out, state_out, B, T, H, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace kairos
