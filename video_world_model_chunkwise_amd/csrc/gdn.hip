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

#include <algorithm>

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
constexpr int TS = CH + 8;      // row stride of the bf16 T tile in the prep kernel
constexpr int ADS = 20;         // row stride of an fp32 diagonal block of A in the prep kernel

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

typedef short s16x4 __attribute__((ext_vector_type(4)));
// Transposed LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane i receives element (i % 4) of the 8-byte pieces addressed by lanes
// 4j + i/4, j = 0..3.  With lane s addressing row k0 + s/4, columns
// c(s % 4) .. c(s % 4) + 3, lane i receives column c(i/4) + i%4 of rows
// k0 .. k0 + 3.
__device__ __forceinline__ uint2 lds_read_tr(const uint16_t* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (s16x4 __attribute__((address_space(3)))*)(p));
  return __builtin_bit_cast(uint2, r);
}

// Raw buffer descriptor: loads at byte offsets >= nbytes return zero and
// stores there are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}

// ---- prep: per (b, h, chunk), independent of the state
//   g_t = sum_{s<=t} log2 a_s            (written out, fp32)
//   A   = strictlower(b_t 2^{g_t - g_i} k_t.k_i)
//   T   = (I + A)^{-1}                   (written out, bf16, unit lower triangular)
// One wave per chunk: the 64 x D key tile stays in registers (it is both
// operands of the Gram product).  T by blocks of 16: diagonal blocks by
// forward substitution, then the 16x16 off-diagonal block of each 32x32
// half, then the lower-left 32x32 block T_LL = -T_H A_HL T_L (block inverse
// of a lower triangular matrix).  Only the forward substitution needs A in
// fp32, so only A's four diagonal blocks go to LDS in fp32; its off-diagonal
// blocks are matrix-product operands (bf16) and sit in the T tile at the
// places their T blocks take later, each read before its T block is written.
// The smaller LDS footprint lets more waves run per CU.
struct PrepSmem {
  float Ad[4][16][ADS];
  uint16_t Tb[CH][TS];
  float g2[CH];
  float bet[CH];
};

template <int D>
__global__ __launch_bounds__(64) void gdn_prep_kernel(const uint16_t* __restrict__ k,
                                                      const float* __restrict__ alpha,
                                                      const float* __restrict__ beta,
                                                      uint16_t* __restrict__ t_out,
                                                      float* __restrict__ g_out, int T, int H,
                                                      int nchunks) {
  constexpr int DS = D / 32;
  __shared__ __attribute__((aligned(16))) PrepSmem sm;
  // Heads vary fastest, and each XCD takes a contiguous range of the
  // (chunk, head) order: the waves of one chunk's heads run together on one
  // XCD, so the per-token rows of k, alpha and beta (all heads of a token are
  // adjacent in memory) are fetched once into that XCD's L2 and shared.
  const int BH = (int)(gridDim.x / nchunks);
  const int lid = xcd_swizzle(blockIdx.x, gridDim.x);
  const int c = lid / BH;
  const int bh = lid % BH;
  const int b = bh / H, h = bh % H;
  const int t0 = c * CH;
  const int valid = min(CH, T - t0);
  const int lane = threadIdx.x, l16 = lane % 16, g = lane / 16;

  // key tile: kr[a][s] = k[t0 + 16a + l16][32s + 8g .. +8] (zero past T)
  const uint32_t tok_bytes = (uint32_t)H * D * 2;
  const auto rk = buf_rsrc(k + (((size_t)b * T + t0) * H + h) * D, (uint32_t)(valid - 1) * tok_bytes + D * 2);
  uint4 kr[4][DS];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int s = 0; s < DS; ++s)
      kr[a][s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rk, (uint32_t)(16 * a + l16) * tok_bytes + (32 * s + 8 * g) * 2, 0, 0));
  {
    const int t = t0 + lane;
    const float av = lane < valid ? alpha[((size_t)b * T + t) * H + h] : 1.f;   // padding: no decay,
    const float bv = lane < valid ? beta[((size_t)b * T + t) * H + h] : 0.f;    // no write
    float x = __log2f(av);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    sm.g2[lane] = x;
    sm.bet[lane] = bv;
    g_out[((size_t)bh * nchunks + c) * CH + lane] = x;
  }
  for (int i = lane; i < CH * TS / 8; i += 64) reinterpret_cast<uint4*>(&sm.Tb[0][0])[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  // A = strictlower(b 2^{dg} K K^T): diagonal tiles in fp32, the others in
  // bf16 in the T tile.  Lane (l16, g) of tile (ti, tj) holds rows
  // 16 ti + 4g + r (r = 0..3) of column 16 tj + l16.
  float4 grow[4], brow[4];
  float gcol[4];
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) {
    grow[ti] = *reinterpret_cast<const float4*>(&sm.g2[16 * ti + 4 * g]);
    brow[ti] = *reinterpret_cast<const float4*>(&sm.bet[16 * ti + 4 * g]);
    gcol[ti] = sm.g2[16 * ti + l16];
  }
#pragma unroll
  for (int task = 0; task < 10; ++task) {
    const int ti = task < 1 ? 0 : task < 3 ? 1 : task < 6 ? 2 : 3;
    const int tj = task - ti * (ti + 1) / 2;
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < DS; ++s) acc = mfma16x16x32(as_bf16x8(kr[ti][s]), as_bf16x8(kr[tj][s]), acc);
    const int col = 16 * tj + l16;
    const float gr[4] = {grow[ti].x, grow[ti].y, grow[ti].z, grow[ti].w};
    const float br[4] = {brow[ti].x, brow[ti].y, brow[ti].z, brow[ti].w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * ti + 4 * g + r;
      const float val = br[r] * __builtin_amdgcn_exp2f(gr[r] - gcol[tj]) * acc[r];
      if (ti == tj) sm.Ad[ti][4 * g + r][l16] = col < row ? val : 0.f;
      else sm.Tb[row][col] = bf16_bits(val);
    }
  }
  __syncthreads();

  // diagonal 16x16 blocks by forward substitution (lane -> block g, column
  // l16), the block's rows of A read into registers first
  {
    const int blk = g, j = l16;
    float a[16][16];
#pragma unroll
    for (int t = 1; t < 16; ++t)
#pragma unroll
      for (int q = 0; q < (t + 3) / 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(&sm.Ad[blk][t][4 * q]);
        a[t][4 * q] = v.x; a[t][4 * q + 1] = v.y; a[t][4 * q + 2] = v.z; a[t][4 * q + 3] = v.w;
      }
    float x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < t; ++i) s4[i % 4] = fmaf(a[t][i], x[i], s4[i % 4]);
      x[t] = ((t == j) ? 1.f : 0.f) - ((s4[0] + s4[1]) + (s4[2] + s4[3]));
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) sm.Tb[16 * blk + t][16 * blk + j] = bf16_bits(x[t]);
  }
  __syncthreads();

  // T_{h1,h0} = -T_{h1,h1} A_{h1,h0} T_{h0,h0} for the two 32x32 halves
  // (K = 16 padded to 32: slots 8g + r <-> k = 4g + r, slots 8g+4.. are zero);
  // the columns of T_{h0,h0} come from transposed reads (4 rows each)
  f32x4 t10[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int h0 = 2 * half, h1 = 2 * half + 1;
    const uint2 av = *reinterpret_cast<const uint2*>(&sm.Tb[16 * h1 + l16][16 * h0 + 4 * g]);   // A_{h1,h0}
    const bf16x8 a = as_bf16x8(av, make_uint2(0, 0));
    const uint2 lo = lds_read_tr(&sm.Tb[16 * h0 + 4 * g + l16 / 4][16 * h0 + 4 * (l16 % 4)]);
    const f32x4 z = mfma16x16x32(a, as_bf16x8(lo, make_uint2(0, 0)), zero4());
    const uint2 tlo = *reinterpret_cast<const uint2*>(&sm.Tb[16 * h1 + l16][16 * h1 + 4 * g]);
    t10[half] = mfma16x16x32(as_bf16x8(tlo, make_uint2(0, 0)),
                             to_bf16x8(z[0], z[1], z[2], z[3], 0.f, 0.f, 0.f, 0.f), zero4());
  }
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.Tb[32 * half + 16 + 4 * g + r][32 * half + l16] = bf16_bits(-t10[half][r]);
  __syncthreads();

  // lower-left 32x32 block: T_LL = -T_H A_HL T_L (column tile tj); rows
  // 8g .. 8g+7 of a column of T_L from two transposed reads
  f32x4 tll[2][2];
#pragma unroll
  for (int tj = 0; tj < 2; ++tj) {
    const uint2 b0 = lds_read_tr(&sm.Tb[8 * g + l16 / 4][16 * tj + 4 * (l16 % 4)]);
    const uint2 b1 = lds_read_tr(&sm.Tb[8 * g + 4 + l16 / 4][16 * tj + 4 * (l16 % 4)]);
    f32x4 z[2];
#pragma unroll
    for (int zi = 0; zi < 2; ++zi) {
      const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.Tb[32 + 16 * zi + l16][8 * g]));   // A_HL
      z[zi] = mfma16x16x32(a, as_bf16x8(b0, b1), zero4());
    }
    const bf16x8 zb = regs_operand(z[0], z[1]);
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
      tll[tj][ti] = mfma16x16x32(row_operand_perm(&sm.Tb[32 + 16 * ti + l16][0], 32, g), zb, zero4());
  }
  // (all reads of the lower-left block's inputs are done before it is written)
#pragma unroll
  for (int tj = 0; tj < 2; ++tj)
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.Tb[32 + 16 * ti + 4 * g + r][16 * tj + l16] = bf16_bits(-tll[tj][ti][r]);
  __syncthreads();

  // write T (64 x 64 bf16, row-major)
  uint16_t* tdst = t_out + ((size_t)bh * nchunks + c) * CH * CH;
#pragma unroll
  for (int u = lane; u < CH * CH / 8; u += 64) {
    const int row = u / 8, cg = u % 8;
    *reinterpret_cast<uint4*>(tdst + row * CH + 8 * cg) = *reinterpret_cast<const uint4*>(&sm.Tb[row][8 * cg]);
  }
}

// ---- scan: per (b, h, 16*NW rows of S), chunks in order
//
// Token order inside LDS.  The products that chain through registers need
// their reduction slots in natural token order: the C registers of 16x16
// tiles 2p and 2p+1 form one operand whose slot 8g + i is token 32p + 8g + i
// when tile 2p row 4g + r holds token 32p + 8g + r and tile 2p+1 row 4g + r
// holds token 32p + 8g + 4 + r.  Every token-major tile (K, Q, V, T, P) is
// therefore staged with token t = 32p + 8g + 4h + r in LDS row
// 32p + 16h + 4g + r, so that the rows of every 16x16 tile are 16
// consecutive LDS rows and each transposed read takes 4 consecutive rows.
//
// State layout: wave w owns rows n_w .. n_w + 15 of S.  S[dt] is a C tile
// whose row 4g + r holds feature (column of S) cb(dt, g) + r with
// cb(2s, g) = 32s + 8g and cb(2s + 1, g) = 32s + 8g + 4, and whose column is
// row n_w + l16 of S; the pair (S[2s], S[2s+1]) is then an operand over 32
// consecutive features in natural order, matching 16-byte reads of K and Q.
//
// Staging: the next chunk's tiles go from HBM straight into the other LDS
// buffer (buffer loads with the LDS flag: lane l of a load writes 16 bytes at
// the load's LDS base + 16 l), so staging costs neither registers nor LDS
// write instructions.  Each buffer is a separate LDS variable so that the
// compiler can tell the in-flight loads from the reads of the current chunk.
// LDS row strides are 16 mod 32 bf16 elements: 16-byte operand reads and
// transposed reads of a 16-row tile then touch distinct banks; padding
// units are filled with copies of real units.
__device__ __forceinline__ int lds_row(int t) {       // token -> LDS row
  return (t & ~31) | ((t & 4) << 2) | ((t & 24) >> 1) | (t & 3);
}
__device__ __forceinline__ int row_token(int row) {   // LDS row -> token
  return (row & ~31) | ((row & 16) >> 2) | ((row & 12) << 1) | (row & 3);
}
__device__ __forceinline__ int s_feature(int dt, int g) {   // cb(dt, g)
  return 32 * (dt / 2) + 8 * g + 4 * (dt % 2);
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;


__device__ __forceinline__ void buf_to_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void buf_to_lds4(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, off, 0, 0, 0);
}
__device__ __forceinline__ void buf_store8(uint2 x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), r, off, 0, 0);
}
// An element offset the compiler must treat as unknown.  LDS-DMA targets
// written as a constant offset into a __shared__ array become a constant
// expression whose generic-to-LDS cast this compiler fails to lower.
__device__ __forceinline__ int opaque_offset(int v) {
  asm volatile("" : "+s"(v));
  return v;
}
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)
// until at most N vector memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// bytes from a chunk's first token to the end of its last valid token row
__device__ __forceinline__ uint32_t chunk_bytes(int T, int c, uint32_t tok_bytes, int D) {
  const int valid = min(CH, T - c * CH);
  return (uint32_t)(valid - 1) * tok_bytes + (uint32_t)D * 2;
}

template <int D, int NW>
struct ScanGeom {
  static constexpr int NR = 16 * NW;                               // S rows per workgroup
  static constexpr int KST = D + 16;                               // K, Q row stride
  static constexpr int VST = NR;                                   // V slice row stride
  static constexpr int OST = NR + 8;                               // O staging row stride
  static constexpr int TST = CH + 16;                              // T, P row stride
  static constexpr int KU = KST / 8, VU = VST / 8, TU = TST / 8;   // 16-byte units per row
  // a tile of 64 rows x U units is exactly U loads of 64 lanes
  // with four compute waves, wave w computes the P tiles of query block w
  // inside its X/Y pass (it keeps that Q block in registers)
  static constexpr bool PM = NW == 4;
};

// One LDS buffer (pointers into separate __shared__ variables).
struct ScanBuf {
  uint16_t* K;
  uint16_t* Q;
  uint16_t* V;
  uint16_t* T;
  float* g2;    // g_t (log2 units), natural token order
  float* gam;   // 2^{g_t}
  float* wts;   // 2^{g_C - g_t}
  float* bet;   // b_t (0 past the sequence)
};

// P tiles: query LDS rows 16a.., key LDS rows 16b..; the 12 tiles with
// floor(a/2) >= floor(b/2) cover the causal part (32-token blocks).
__device__ __forceinline__ void p_tile_of(int task, int& a, int& b) {
  a = task < 4 ? task / 2 : 2 + (task - 4) / 4;
  b = task < 4 ? task % 2 : (task - 4) % 4;
}

template <int D, int NW>
struct ScanCtx {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* beta;
  const uint16_t* t_in;
  const float* g_in;
  uint16_t* out;
  size_t head0;          // element offset of (b, t = 0, h)
  size_t chunk_elems;    // elements per 64 tokens of the [B][T][H][D] tensors
  size_t tg0;            // chunk 0 of this head in the T / g workspace (in chunks)
  size_t beta0;          // element offset of (b, t = 0, h) in beta
  int T, H, nchunks, n_base, wave;
  uint32_t tok_bytes;
  bool vzero;            // transition rows: V is read as zero (empty buffer range)
};

// Per-lane byte offsets of the loader wave's loads inside a chunk: load m of
// a tile fills 16-byte units 64 m .. 64 m + 63 (row = unit / units per row).
// Each of the NW loader waves issues loads m = lw, lw + NW, ... of each tile.
// The loader index is a compile-time constant, so that every load of a
// wave is unconditional and the compiler's waits for LDS data written by
// these loads count exactly the loads issued after them.
template <int D, int NW, int LW>
struct ScanLoadOffs {
  static constexpr int lw = LW;      // loader index 0 .. NW-1
  static constexpr int KJ = (ScanGeom<D, NW>::KU + NW - 1) / NW;
  static constexpr int VJ = (ScanGeom<D, NW>::VU + NW - 1) / NW;
  static constexpr int TJ = (ScanGeom<D, NW>::TU + NW - 1) / NW;
  uint32_t kq[KJ];
  uint32_t v[VJ];
  uint32_t t[TJ];
  // loads m = lw, lw + NW, ... < U of a tile of U loads
  static constexpr int share(int U) { return U > LW ? (U - 1 - LW) / NW + 1 : 0; }
  // loads of the Q/V/T batch (no Q without outputs)
  template <bool OUT>
  static constexpr int qvt_loads() {
    return (OUT ? share(ScanGeom<D, NW>::KU) : 0) + share(ScanGeom<D, NW>::VU) + share(ScanGeom<D, NW>::TU);
  }
};

// Loads of chunk c into LDS buffer bf, this loader wave's share (loads
// m = lw, lw + NW, ... of each tile).  Two batches per chunk: K with g and b
// (needed through the whole chunk), and Q, V, T (read before the middle of
// the chunk, so they are fetched one chunk earlier into the buffer that the
// chunk two steps back has released).
template <int D, int NW, int LW>
__device__ __forceinline__ void scan_issue_k(const ScanCtx<D, NW>& x, const ScanLoadOffs<D, NW, LW>& lo,
                                             const ScanBuf& bf, int c) {
  using G = ScanGeom<D, NW>;
  using L = ScanLoadOffs<D, NW, LW>;
  const int lane = threadIdx.x % 64;
  const size_t e0 = x.head0 + (size_t)c * x.chunk_elems;
  const auto rk = buf_rsrc(x.k + e0, chunk_bytes(x.T, c, x.tok_bytes, D));
  if constexpr (LW == 0) {
    const int valid = min(CH, x.T - c * CH);
    const auto rg = buf_rsrc(x.g_in + (x.tg0 + c) * CH, CH * 4);
    const auto rb = buf_rsrc(x.beta + x.beta0 + (size_t)c * CH * x.H, (uint32_t)((valid - 1) * x.H + 1) * 4);
    buf_to_lds4(rg, bf.g2, lane * 4);
    buf_to_lds4(rb, bf.bet, (uint32_t)lane * x.H * 4);
  }
#pragma unroll
  for (int j = 0; j < L::KJ; ++j) {
    const int m = LW + NW * j;
    if (m < G::KU) buf_to_lds16(rk, bf.K + opaque_offset(512 * m), lo.kq[j]);
  }
}

template <int D, int NW, int LW, bool OUT>
__device__ __forceinline__ void scan_issue_qvt(const ScanCtx<D, NW>& x, const ScanLoadOffs<D, NW, LW>& lo,
                                               const ScanBuf& bf, int c) {
  using G = ScanGeom<D, NW>;
  using L = ScanLoadOffs<D, NW, LW>;
  const size_t e0 = x.head0 + (size_t)c * x.chunk_elems;
  const uint32_t nrec = chunk_bytes(x.T, c, x.tok_bytes, D);
  const auto rq = buf_rsrc(x.q + e0, nrec);
  const auto rv = buf_rsrc(x.v + e0 + x.n_base, x.vzero ? 0u : nrec);
  const auto rt = buf_rsrc(x.t_in + (x.tg0 + c) * CH * CH, CH * CH * 2);
#pragma unroll
  for (int j = 0; j < L::TJ; ++j) {
    const int m = LW + NW * j;
    if (m < G::TU) buf_to_lds16(rt, bf.T + opaque_offset(512 * m), lo.t[j]);
  }
#pragma unroll
  for (int j = 0; j < L::VJ; ++j) {
    const int m = LW + NW * j;
    if (m < G::VU) buf_to_lds16(rv, bf.V + opaque_offset(512 * m), lo.v[j]);
  }
  if constexpr (OUT) {
#pragma unroll
    for (int j = 0; j < L::KJ; ++j) {
      const int m = LW + NW * j;
      if (m < G::KU) buf_to_lds16(rq, bf.Q + opaque_offset(512 * m), lo.kq[j]);
    }
  }
}

// 2^{g} and 2^{g_C - g} of a staged chunk (wave 0, after its loads landed)
__device__ __forceinline__ void scan_decays(const ScanBuf& bf) {
  const int lane = threadIdx.x % 64;
  const float gv = bf.g2[lane];
  const float gl = bf.g2[CH - 1];
  bf.gam[lane] = __builtin_amdgcn_exp2f(gv);
  bf.wts[lane] = __builtin_amdgcn_exp2f(gl - gv);
}

// O of chunk c from the staging tile (token-natural rows, this workgroup's
// NR columns) to HBM: 2 stores of 16 bytes per lane per loader wave.  With
// store = false the stores go to an empty range (nothing is written), so
// that every chunk issues the same number of memory operations.
template <int D, int NW, int LW>
__device__ __forceinline__ void scan_store_o(const ScanCtx<D, NW>& x, const uint16_t* Os, int c, bool store) {
  using G = ScanGeom<D, NW>;
  constexpr int UPR = G::NR / 8;            // 16-byte units per row
  const int lane = threadIdx.x % 64;
  uint4 d[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int U = 64 * (LW + NW * j) + lane;
    d[j] = *reinterpret_cast<const uint4*>(Os + (U / UPR) * G::OST + (U % UPR) * 8);
  }
  const auto ro = buf_rsrc(x.out + x.head0 + (size_t)c * x.chunk_elems + x.n_base,
                           store ? chunk_bytes(x.T, c, x.tok_bytes, G::NR) : 0u);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int U = 64 * (LW + NW * j) + lane;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, d[j]), ro,
                                           (uint32_t)(U / UPR) * x.tok_bytes + (U % UPR) * 16, 0, 0);
  }
}

// One chunk of a compute wave: reads buffer cb.  Without outputs (OUT
// false) only the state is advanced: no Q, no P, no O.
template <int D, int NW, bool OUT>
__device__ __forceinline__ void scan_chunk(const ScanCtx<D, NW>& x, const ScanBuf& cb,
                                           uint16_t* Pb, uint16_t* Os, f32x4 (&S)[D / 16], int c) {
  using G = ScanGeom<D, NW>;
  constexpr int DT = D / 16, DS = D / 32;
  constexpr int KST = G::KST, VST = G::VST, TST = G::TST;
  const int lane = threadIdx.x % 64, l16 = lane % 16, g = lane / 16;
  const int wave = x.wave;

  // LDS reads run ahead of the products that consume them: each step issues
  // the next step's reads before its own products (rings of two register
  // sets), and the scheduling fences keep that order.
  // ---- P = lower(2^{g_t - g_i} q_t . k_i), as tiles of K Q^T: lane holds
  //      keys i0 .. i0+3 (consecutive tokens) of query t
  constexpr int NTASK = 12 / NW;
  if constexpr (OUT && !G::PM) {
    uint4 pk[2][DS], pq[2][DS];
    float gt[2];
    float4 gi[2];
    int pt[2], pi0[2], prow[2];
#define KAIROS_P_LOAD(j, buf)                                                              \
    {                                                                                      \
      int a_, b_;                                                                          \
      p_tile_of(wave + NW * (j), a_, b_);                                                  \
      const uint16_t* krow = cb.K + (16 * b_ + l16) * KST + 8 * g;                         \
      const uint16_t* qrow = cb.Q + (16 * a_ + l16) * KST + 8 * g;                         \
      _Pragma("unroll") for (int s = 0; s < DS; ++s) {                                     \
        pk[buf][s] = *reinterpret_cast<const uint4*>(krow + 32 * s);                       \
        pq[buf][s] = *reinterpret_cast<const uint4*>(qrow + 32 * s);                       \
      }                                                                                    \
      pt[buf] = row_token(16 * a_ + l16);                                                  \
      pi0[buf] = row_token(16 * b_ + 4 * g);                                               \
      prow[buf] = 16 * a_ + l16;                                                           \
      gt[buf] = cb.g2[pt[buf]];                                                            \
      gi[buf] = *reinterpret_cast<const float4*>(cb.g2 + pi0[buf]);                        \
    }
    KAIROS_P_LOAD(0, 0);
#pragma unroll
    for (int j = 0; j < NTASK; ++j) {
      const int cur_b = j & 1;
      if (j + 1 < NTASK) KAIROS_P_LOAD(j + 1, cur_b ^ 1);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < DS; ++s) acc = mfma16x16x32(as_bf16x8(pk[cur_b][s]), as_bf16x8(pq[cur_b][s]), acc);
      const int t = pt[cur_b], i0 = pi0[cur_b];
      const float gtv = gt[cur_b];
      const float4 giv = gi[cur_b];
      const float p0 = i0 <= t ? __builtin_amdgcn_exp2f(gtv - giv.x) * acc[0] : 0.f;
      const float p1 = i0 + 1 <= t ? __builtin_amdgcn_exp2f(gtv - giv.y) * acc[1] : 0.f;
      const float p2 = i0 + 2 <= t ? __builtin_amdgcn_exp2f(gtv - giv.z) * acc[2] : 0.f;
      const float p3 = i0 + 3 <= t ? __builtin_amdgcn_exp2f(gtv - giv.w) * acc[3] : 0.f;
      *reinterpret_cast<uint2*>(Pb + prow[cur_b] * TST + i0) = pack_bf16x4(p0, p1, p2, p3);
      __builtin_amdgcn_sched_barrier(0);
    }
#undef KAIROS_P_LOAD
  }

  // ---- state-dependent products for this wave's 16 rows of S
  // X = K S^T (tile tt row 4g + r: token 32(tt/2) + 8g + 4(tt%2) + r, column n_w + l16)
  // Y^T = S Q^T (row n_w + 4g + r, column: token row_token(16 tt + l16))
  f32x4 X[4], Y[4];
  uint2 vv[4];
  float4 bt[4], gm[4];
  uint4 tr[6];
  {
    uint4 xk[2][DS], xq[2][DS];
#define KAIROS_XY_LOAD(tt, buf)                                                            \
    {                                                                                      \
      const uint16_t* krow = cb.K + (16 * (tt) + l16) * KST + 8 * g;                       \
      const uint16_t* qrow = cb.Q + (16 * (tt) + l16) * KST + 8 * g;                       \
      _Pragma("unroll") for (int s = 0; s < DS; ++s) {                                     \
        xk[buf][s] = *reinterpret_cast<const uint4*>(krow + 32 * s);                       \
        if constexpr (OUT) xq[buf][s] = *reinterpret_cast<const uint4*>(qrow + 32 * s);    \
      }                                                                                    \
    }
    KAIROS_XY_LOAD(0, 0);
    // PM: query block `wave` of P = lower(2^{g_t - g_i} q_t . k_i); tile
    // (wave, tt) for the key blocks tt of the same or an earlier 32-token half
    uint4 qw[DS];
    int p_t = 0;
    float p_gt = 0.f;
    if constexpr (OUT && G::PM) {
      const uint16_t* qrow = cb.Q + (16 * wave + l16) * KST + 8 * g;
#pragma unroll
      for (int s = 0; s < DS; ++s) qw[s] = *reinterpret_cast<const uint4*>(qrow + 32 * s);
      p_t = row_token(16 * wave + l16);
      p_gt = cb.g2[p_t];
    }
    bf16x8 Sop[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) Sop[s] = regs_operand(S[2 * s], S[2 * s + 1]);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int cur_b = tt & 1;
      float4 p_gi = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (OUT && G::PM) p_gi = *reinterpret_cast<const float4*>(cb.g2 + row_token(16 * tt + 4 * g));
      if (tt + 1 < 4) {
        KAIROS_XY_LOAD(tt + 1, cur_b ^ 1);
      } else {
        // operands of R and E
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int tau0 = 32 * (u / 2) + 8 * g + 4 * (u % 2);
          vv[u] = lds_read_tr(cb.V + (16 * u + 4 * g + l16 / 4) * VST + 16 * wave + 4 * (l16 % 4));
          bt[u] = *reinterpret_cast<const float4*>(cb.bet + tau0);
          gm[u] = *reinterpret_cast<const float4*>(cb.gam + tau0);
          tr[u] = *reinterpret_cast<const uint4*>(cb.T + (16 * u + l16) * TST + 8 * g);
        }
        tr[4] = *reinterpret_cast<const uint4*>(cb.T + (32 + l16) * TST + 32 + 8 * g);
        tr[5] = *reinterpret_cast<const uint4*>(cb.T + (48 + l16) * TST + 32 + 8 * g);
      }
      __builtin_amdgcn_sched_barrier(0);
      X[tt] = zero4();
      Y[tt] = zero4();
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        X[tt] = mfma16x16x32(as_bf16x8(xk[cur_b][s]), Sop[s], X[tt]);
        if constexpr (OUT) Y[tt] = mfma16x16x32(Sop[s], as_bf16x8(xq[cur_b][s]), Y[tt]);
      }
      if constexpr (OUT && G::PM) {
        if (wave >= 2 * (tt / 2)) {
          f32x4 acc = zero4();
#pragma unroll
          for (int s = 0; s < DS; ++s) acc = mfma16x16x32(as_bf16x8(xk[cur_b][s]), as_bf16x8(qw[s]), acc);
          const int i0 = row_token(16 * tt + 4 * g);
          const float p0 = i0 <= p_t ? __builtin_amdgcn_exp2f(p_gt - p_gi.x) * acc[0] : 0.f;
          const float p1 = i0 + 1 <= p_t ? __builtin_amdgcn_exp2f(p_gt - p_gi.y) * acc[1] : 0.f;
          const float p2 = i0 + 2 <= p_t ? __builtin_amdgcn_exp2f(p_gt - p_gi.z) * acc[2] : 0.f;
          const float p3 = i0 + 3 <= p_t ? __builtin_amdgcn_exp2f(p_gt - p_gi.w) * acc[3] : 0.f;
          *reinterpret_cast<uint2*>(Pb + (16 * wave + l16) * TST + i0) = pack_bf16x4(p0, p1, p2, p3);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#undef KAIROS_XY_LOAD
  }
  // K^T operands of the first two S-update steps and the decay weights go
  // out before R and E
  uint2 kt[2][4];
  float gmo[4];
  float4 w4[4];
  const uint16_t* kcol = cb.K + (4 * g + l16 / 4) * KST;
#define KAIROS_KT_LOAD(dt, buf)                                                            \
  {                                                                                        \
    const uint16_t* kc = kcol + s_feature(dt, l16 % 4);                                    \
    kt[buf][0] = lds_read_tr(kc);                                                          \
    kt[buf][1] = lds_read_tr(kc + 16 * KST);                                               \
    kt[buf][2] = lds_read_tr(kc + 32 * KST);                                               \
    kt[buf][3] = lds_read_tr(kc + 48 * KST);                                               \
  }
  KAIROS_KT_LOAD(0, 0);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    gmo[tt] = cb.gam[row_token(16 * tt + l16)];
    w4[tt] = *reinterpret_cast<const float4*>(cb.wts + 32 * (tt / 2) + 8 * g + 4 * (tt % 2));
  }
  const float gC = cb.gam[CH - 1];
  __builtin_amdgcn_sched_barrier(0);
  // R = b (V - 2^g X);  E = T R (rows as X; T is lower triangular)
  f32x4 E[4];
  {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      X[tt][0] = bt[tt].x * (bf16_to_f32(lo16(vv[tt].x)) - gm[tt].x * X[tt][0]);
      X[tt][1] = bt[tt].y * (bf16_to_f32(hi16(vv[tt].x)) - gm[tt].y * X[tt][1]);
      X[tt][2] = bt[tt].z * (bf16_to_f32(lo16(vv[tt].y)) - gm[tt].z * X[tt][2]);
      X[tt][3] = bt[tt].w * (bf16_to_f32(hi16(vv[tt].y)) - gm[tt].w * X[tt][3]);
    }
    const bf16x8 Rop0 = regs_operand(X[0], X[1]);
    const bf16x8 Rop1 = regs_operand(X[2], X[3]);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) E[tt] = mfma16x16x32(as_bf16x8(tr[tt]), Rop0, zero4());
    E[2] = mfma16x16x32(as_bf16x8(tr[4]), Rop1, E[2]);
    E[3] = mfma16x16x32(as_bf16x8(tr[5]), Rop1, E[3]);
  }
  lds_barrier();                      // P complete; this chunk's Q, V, T released

  // O^T = 2^g Y^T + E^T P^T;  S <- 2^{g_C} S + K^T diag(w) E
  {
    uint4 po[6];
    if constexpr (OUT) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) po[tt] = *reinterpret_cast<const uint4*>(Pb + (16 * tt + l16) * TST + 8 * g);
      po[4] = *reinterpret_cast<const uint4*>(Pb + (32 + l16) * TST + 32 + 8 * g);
      po[5] = *reinterpret_cast<const uint4*>(Pb + (48 + l16) * TST + 32 + 8 * g);
    }
    KAIROS_KT_LOAD(1, 1);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 WE[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      WE[tt] = f32x4{w4[tt].x * E[tt][0], w4[tt].y * E[tt][1], w4[tt].z * E[tt][2], w4[tt].w * E[tt][3]};
    const bf16x8 WEop0 = regs_operand(WE[0], WE[1]);
    const bf16x8 WEop1 = regs_operand(WE[2], WE[3]);
    if constexpr (OUT) {
      const bf16x8 Eop0 = regs_operand(E[0], E[1]);
      const bf16x8 Eop1 = regs_operand(E[2], E[3]);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        f32x4 o = f32x4{gmo[tt] * Y[tt][0], gmo[tt] * Y[tt][1], gmo[tt] * Y[tt][2], gmo[tt] * Y[tt][3]};
        o = mfma16x16x32(Eop0, as_bf16x8(po[tt]), o);
        if (tt >= 2) o = mfma16x16x32(Eop1, as_bf16x8(po[tt + 2]), o);
        *reinterpret_cast<uint2*>(Os + row_token(16 * tt + l16) * G::OST + 16 * wave + 4 * g) =
            pack_bf16x4(o[0], o[1], o[2], o[3]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int cur_b = dt & 1;
      // kt[cur_b] holds step dt; refill the other set with step dt + 1 once it is free
      f32x4 sv = f32x4{gC * S[dt][0], gC * S[dt][1], gC * S[dt][2], gC * S[dt][3]};
      sv = mfma16x16x32(as_bf16x8(kt[cur_b][0], kt[cur_b][1]), WEop0, sv);
      sv = mfma16x16x32(as_bf16x8(kt[cur_b][2], kt[cur_b][3]), WEop1, sv);
      S[dt] = sv;
      if (dt + 2 < DT) KAIROS_KT_LOAD(dt + 2, cur_b);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#undef KAIROS_KT_LOAD
  lds_barrier();                      // the next chunk has landed (loader wave)
}

// Loader wave, one chunk c (buffer cb; nb is the other buffer): K, g, b of
// chunk c+1 into nb, then O of chunk c-1 from the staging tile to HBM (the
// compute waves overwrite it after the middle barrier); after that barrier,
// when chunk c no longer reads its Q, V, T, the Q/V/T batch of chunk c+2 into
// cb; 2^{g} and 2^{g_C - g} of chunk c+1.  Before the end barrier everything
// but the newest batch has landed.  Two barriers per chunk, as in the compute
// waves.
template <int D, int NW, int LW, bool OUT>
__device__ __forceinline__ void scan_load_chunk(const ScanCtx<D, NW>& x, const ScanLoadOffs<D, NW, LW>& lo,
                                                const ScanBuf& cb, const ScanBuf& nb, const uint16_t* Os,
                                                int c) {
  using L = ScanLoadOffs<D, NW, LW>;
  const bool more1 = c + 1 < x.nchunks, more2 = c + 2 < x.nchunks;
  if (more1) scan_issue_k<D, NW, LW>(x, lo, nb, c + 1);
  if constexpr (OUT) scan_store_o<D, NW, LW>(x, Os, c - 1, c > 0);
  lds_barrier();
  if constexpr (LW == 0) {
    if (more1) {
      // g and b of chunk c+1 (issued before its K loads and the two O stores)
      wait_vmem_le<L::share(ScanGeom<D, NW>::KU) + (OUT ? 2 : 0)>();
      scan_decays(nb);
    }
  }
  if (more2) {
    scan_issue_qvt<D, NW, LW, OUT>(x, lo, cb, c + 2);
    wait_vmem_le<L::template qvt_loads<OUT>()>();           // all but the batch just issued
  } else {
    wait_vmem();
  }
  lds_barrier();
}

// One loader wave: its load offsets, the first two chunks, then one
// scan_load_chunk per chunk.
template <int D, int NW, int LW, bool OUT>
__device__ __forceinline__ void scan_loader(const ScanCtx<D, NW>& x, const ScanBuf& B0, const ScanBuf& B1,
                                            const uint16_t* Os) {
  using G = ScanGeom<D, NW>;
  using L = ScanLoadOffs<D, NW, LW>;
  constexpr int NR = G::NR;
  const int lane = threadIdx.x % 64;
  L lo;
#pragma unroll
  for (int j = 0; j < L::KJ; ++j) {
    const int U = 64 * (LW + NW * j) + lane;
    lo.kq[j] = (uint32_t)row_token(U / G::KU) * x.tok_bytes + (U % G::KU) % (D / 8) * 16;
  }
#pragma unroll
  for (int j = 0; j < L::VJ; ++j) {
    const int U = 64 * (LW + NW * j) + lane;
    lo.v[j] = (uint32_t)row_token(U / G::VU) * x.tok_bytes + (U % G::VU) % (NR / 8) * 16;
  }
#pragma unroll
  for (int j = 0; j < L::TJ; ++j) {
    const int U = 64 * (LW + NW * j) + lane;
    lo.t[j] = (uint32_t)row_token(U / G::TU) * (CH * 2) + (U % G::TU) % 8 * 16;
  }
  if (x.nchunks > 0) {
    scan_issue_k<D, NW, LW>(x, lo, B0, 0);
    scan_issue_qvt<D, NW, LW, OUT>(x, lo, B0, 0);
    if (x.nchunks > 1) scan_issue_qvt<D, NW, LW, OUT>(x, lo, B1, 1);
    wait_vmem();
    if constexpr (LW == 0) scan_decays(B0);
  }
  lds_barrier();
  for (int c = 0; c < x.nchunks; c += 2) {
    scan_load_chunk<D, NW, LW, OUT>(x, lo, B0, B1, Os, c);
    if (c + 1 < x.nchunks) scan_load_chunk<D, NW, LW, OUT>(x, lo, B1, B0, Os, c + 1);
  }
  if constexpr (OUT) {
    if (x.nchunks > 0) scan_store_o<D, NW, LW>(x, Os, x.nchunks - 1, true);
  }
}

// Arguments of a scan launch.  The sequence of each (b, h) is cut into nsegs
// segments of seg_chunks chunks (one segment: the plain scan); a launch runs
// nseg_launch segments (from segment 0), each as `tiles` row tiles of 16 NW
// rows.  Tiles below D / (16 NW) advance rows of the state S; tiles above
// advance rows of the segment's transition M (the same recurrence with v = 0,
// started from the identity), so that S_end = S_start M + S_end(from zero);
// segment 0 has no transition tiles.
//   start state of segment j (state rows): init_seg[bh][j] when init_seg is
//     given, else state_in for j = 0 (NULL: zero), else zero;
//   end state: the last segment of the sequence -> state_out (NULL: dropped);
//     other segments -> fin_seg[bh][j + 1] (NULL: dropped); transition rows
//     -> fin_trans[bh][j].
// The per-(b, h) segment arrays hold nsegs slots of D x D fp32.
struct GdnScanArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* beta;
  const uint16_t* t_in;
  const float* g_in;
  uint16_t* out;
  const float* state_in;
  float* state_out;
  const float* init_seg;
  float* fin_seg;
  float* fin_trans;
  int B, T, H, nchunks;
  int seg_chunks, nsegs, nseg_launch, tiles;
};

// Workgroup: NW compute waves (16 rows of S each) and NW loader waves that
// stream the next chunk into the other LDS buffer (each SIMD runs one of
// each).  The double-buffered LDS tiles allow one workgroup per CU.
// Workgroups per (b, h) of a scan launch over nseg segments of `tiles` row
// tiles each, nt of them state tiles: the first segment has no transition tiles.
__host__ __device__ constexpr int scan_tiles_per_bh(int nseg, int tiles, int nt) {
  return nseg * tiles - (tiles - nt);
}

template <int D, int NW, bool OUT>
__global__ __launch_bounds__(128 * NW) void gdn_scan_kernel(const GdnScanArgs a) {
  using G = ScanGeom<D, NW>;
  constexpr int NR = G::NR;
  constexpr int NT = D / NR;          // workgroups per head and segment (state rows)
  constexpr int DT = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t K0[CH * G::KST], K1[CH * G::KST];
  __shared__ __attribute__((aligned(16))) uint16_t Q0[CH * G::KST], Q1[CH * G::KST];
  __shared__ __attribute__((aligned(16))) uint16_t V0[CH * G::VST], V1[CH * G::VST];
  __shared__ __attribute__((aligned(16))) uint16_t T0[CH * G::TST], T1[CH * G::TST];
  __shared__ __attribute__((aligned(16))) uint16_t Pb[CH * G::TST];
  __shared__ __attribute__((aligned(16))) uint16_t Os[CH * G::OST];
  __shared__ __attribute__((aligned(16))) float g0[CH], g1[CH], gam0[CH], gam1[CH];
  __shared__ __attribute__((aligned(16))) float w0[CH], w1[CH], b0[CH], b1[CH];
  const ScanBuf B0{K0, Q0, V0, T0, g0, gam0, w0, b0};
  const ScanBuf B1{K1, Q1, V1, T1, g1, gam1, w1, b1};

  // (b, h) outermost, then segment, then row tile: the tiles of one segment
  // are adjacent and share an XCD (and its L2) for the common K, Q, T reads.
  // The first segment starts from a given state, so it has state tiles only
  // (no transition tiles are launched for it: idle workgroups would share
  // compute units with working ones).
  const int lid = xcd_swizzle(blockIdx.x, gridDim.x);
  const int per_bh = scan_tiles_per_bh(a.nseg_launch, a.tiles, NT);
  const int bh = lid / per_bh;
  if (bh >= a.B * a.H) return;
  const int local = lid % per_bh;
  const int j = local < NT ? 0 : 1 + (local - NT) / a.tiles;
  const int tile = local < NT ? local : (local - NT) % a.tiles;
  const bool trans = tile >= NT;
  const int b = bh / a.H, h = bh % a.H;
  const int c0 = j * a.seg_chunks;
  const int nch = max(0, min(a.seg_chunks, a.nchunks - c0));

  const int lane = threadIdx.x % 64, l16 = lane % 16, g = lane / 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);

  ScanCtx<D, NW> x;
  x.q = a.q; x.k = a.k; x.v = a.v; x.beta = a.beta; x.t_in = a.t_in; x.g_in = a.g_in; x.out = a.out;
  x.T = a.T - c0 * CH; x.H = a.H;
  x.nchunks = nch;
  x.n_base = (tile % NT) * NR;
  x.wave = wave;
  x.tok_bytes = (uint32_t)a.H * D * 2;
  x.chunk_elems = (size_t)CH * a.H * D;
  x.head0 = ((size_t)b * a.T * a.H + h) * D + (size_t)c0 * x.chunk_elems;
  x.tg0 = (size_t)bh * a.nchunks + c0;
  x.beta0 = (size_t)b * a.T * a.H + h + (size_t)c0 * CH * a.H;
  x.vzero = trans;

  if (wave >= NW) {                   // ---- loader waves
    const int lw = wave - NW;
    if (lw == 0) {
      scan_loader<D, NW, 0, OUT>(x, B0, B1, Os);
    } else if constexpr (NW > 1) {
      if (lw == 1) {
        scan_loader<D, NW, 1, OUT>(x, B0, B1, Os);
      } else if constexpr (NW > 2) {
        if (lw == 2) scan_loader<D, NW, 2, OUT>(x, B0, B1, Os);
        else scan_loader<D, NW, 3, OUT>(x, B0, B1, Os);
      }
    }
    return;
  }

  // ---- compute waves
  const int n_w = x.n_base + 16 * wave;     // first row (of S or M) of this wave
  const size_t slot = (size_t)D * D;
  const float* sinit = nullptr;
  if (!trans) {
    if (a.init_seg) sinit = a.init_seg + ((size_t)bh * a.nsegs + j) * slot;
    else if (j == 0) sinit = a.state_in;
  }
  float* sfin = nullptr;
  if (trans) {
    if (a.fin_trans) sfin = a.fin_trans + ((size_t)bh * a.nsegs + j) * slot;
  } else if (j == a.nsegs - 1) {
    sfin = a.state_out ? a.state_out + (size_t)bh * slot : nullptr;
  } else if (a.fin_seg) {
    sfin = a.fin_seg + ((size_t)bh * a.nsegs + j + 1) * slot;
  }

  f32x4 S[DT];
  if (trans) {                        // M starts as the identity: row n is e_n
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[dt][r] = (s_feature(dt, g) + r == n_w + l16) ? 1.f : 0.f;
  } else if (sinit) {
    const float* src = sinit + (a.init_seg ? 0 : (size_t)bh * slot) + (size_t)(n_w + l16) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const float4 s4 = *reinterpret_cast<const float4*>(src + s_feature(dt, g));
      S[dt] = f32x4{s4.x, s4.y, s4.z, s4.w};
    }
  } else {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) S[dt] = zero4();
  }
  lds_barrier();                      // chunk 0 has landed

  for (int c = 0; c < x.nchunks; c += 2) {
    scan_chunk<D, NW, OUT>(x, B0, Pb, Os, S, c);
    if (c + 1 < x.nchunks) scan_chunk<D, NW, OUT>(x, B1, Pb, Os, S, c + 1);
  }

  if (sfin) {
    float* dst = sfin + (size_t)(n_w + l16) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(dst + s_feature(dt, g)) = make_float4(S[dt][0], S[dt][1], S[dt][2], S[dt][3]);
  }
}

// Segment starts from the pass over segments: slot 0 <- state_in (zero when
// NULL); for j = 1 .. nsegs-2, slot j+1 (holding the end state of segment j
// from a zero start) <- slot j * M_j + slot j+1, the affine map of the
// recurrence over segment j applied to its true start.  fp32, one workgroup
// per (b, h, 16 rows of S): rows of S are independent under the map.  The
// next transition is fetched into registers while the current step runs and
// then stored to the other LDS buffer.
template <int D>
__global__ __launch_bounds__(512) void gdn_seg_combine_kernel(const float* state_in, float* starts,
                                                              const float* trans, int nsegs) {
  constexpr int RB = 16;              // rows per workgroup
  constexpr int CPT = RB * D / 512;   // columns per thread
  constexpr int MV = D * D / 4 / 512; // float4 of a transition per thread
  __shared__ __attribute__((aligned(16))) float Ml[2][D * D];
  __shared__ __attribute__((aligned(16))) float Sl[RB * D];
  const int bh = blockIdx.x / (D / RB), r0 = (blockIdx.x % (D / RB)) * RB;
  const size_t slot = (size_t)D * D;
  float* base = starts + (size_t)bh * nsegs * slot;
  const float* tr = trans + (size_t)bh * nsegs * slot;
  const int tid = threadIdx.x, row = tid / (D / CPT), col = (tid % (D / CPT)) * CPT;
  for (int i = tid; i < RB * D; i += 512) {
    const float v = state_in ? state_in[(size_t)bh * slot + (size_t)r0 * D + i] : 0.f;
    base[(size_t)r0 * D + i] = v;
  }
  if (nsegs < 3) return;
  float4 mr[MV];
#pragma unroll
  for (int u = 0; u < MV; ++u) mr[u] = reinterpret_cast<const float4*>(tr + slot)[tid + 512 * u];
#pragma unroll
  for (int u = 0; u < MV; ++u) reinterpret_cast<float4*>(Ml[0])[tid + 512 * u] = mr[u];
  for (int i = tid; i < RB * D / 4; i += 512)
    reinterpret_cast<float4*>(Sl)[i] = reinterpret_cast<const float4*>(base + slot + (size_t)r0 * D)[i];
  __syncthreads();
  for (int jj = 1; jj + 1 < nsegs; ++jj) {
    const bool more = jj + 2 < nsegs;
    if (more) {
#pragma unroll
      for (int u = 0; u < MV; ++u) mr[u] = reinterpret_cast<const float4*>(tr + (size_t)(jj + 1) * slot)[tid + 512 * u];
    }
    const float* Mc = Ml[(jj - 1) & 1];
    float* cur = base + (size_t)(jj + 1) * slot + (size_t)(r0 + row) * D + col;
    float acc[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) acc[u] = cur[u];
#pragma unroll 8
    for (int m = 0; m < D; ++m) {
      const float sv = Sl[row * D + m];
#pragma unroll
      for (int u = 0; u < CPT; ++u) acc[u] = fmaf(sv, Mc[m * D + col + u], acc[u]);
    }
#pragma unroll
    for (int u = 0; u < CPT; ++u) cur[u] = acc[u];
    __syncthreads();                  // every read of Sl and of this step's M done
#pragma unroll
    for (int u = 0; u < CPT; ++u) Sl[row * D + col + u] = acc[u];
    if (more) {
#pragma unroll
      for (int u = 0; u < MV; ++u) reinterpret_cast<float4*>(Ml[jj & 1])[tid + 512 * u] = mr[u];
    }
    __syncthreads();
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

// Segments of the scan over time (1: the plain scan).  With few (b, h) the
// plain scan occupies few compute units for the whole sequence; splitting the
// sequence into P segments runs P - 1 of them from known starts (zero state
// and identity transition, without outputs) in a first pass, combines the
// segment maps, and then all P with their true start states and outputs.
// P minimises a cost model of the two passes and the combine, from the shape
// alone (so that workspace sizes do not depend on the device): a pass of w
// workgroups on 256 compute units runs ceil(w / 256) rounds (a compute unit
// holding two workgroups runs each at about half speed), each round L chunks
// long at a per-chunk time that is the larger of a latency term and a term
// growing with the round's workgroups (memory traffic).  Constants in
// microseconds, fitted to kairos_gdn_fwd times on MI355X over B H in
// {2 .. 64}, T in {4096 .. 65536} and P in {1 .. 16}: the model's choice is
// within 0.5% of the fastest P on every measured shape.
int gdn_segments(int B, int H, int T, int D) {
  const long bh = (long)B * H;
  const long n = (T + CH - 1) / CH;
  if (n < 64 || D % 64 != 0) return 1;
  const long nt = D / 64;                              // state-row workgroups per (b, h)
  constexpr long kCus = 256;
  constexpr double kLat1 = 0.896, kPerWg1 = 3.93e-3;   // first pass (no outputs)
  constexpr double kLat2 = 1.92, kPerWg2 = 8.65e-3;    // second pass, plain scan
  constexpr double kCombineStep = 5.44;
  auto pass = [](long w, long L, double lat, double per_wg) {
    const long full = w / kCus, rest = w % kCus;
    double t = (double)full * std::max(lat, kCus * per_wg);
    if (rest > 0) t += std::max(lat, (double)rest * per_wg);
    return t * (double)L;
  };
  double best = pass(bh * nt, n, kLat2, kPerWg2);
  int best_p = 1;
  for (int P = 2; P <= 16; ++P) {
    const long L = (n + P - 1) / P;
    if ((P - 1) * L >= n) continue;                    // empty last segment
    const double t = pass(bh * nt * (2 * P - 3), L, kLat1, kPerWg1) + pass(bh * nt * P, L, kLat2, kPerWg2) +
                     kCombineStep * (P - 2) * (1.0 + (double)(bh * (D / 16)) / kCus);
    if (t < best) {
      best = t;
      best_p = P;
    }
  }
  return best_p;
}

namespace {
struct GdnWs {
  size_t t, g, starts, trans, total;
};
GdnWs gdn_ws_layout(int B, int T, int H, int D) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t nchunks = (size_t)(T + CH - 1) / CH;
  const size_t bh = (size_t)B * H;
  const int P = gdn_segments(B, H, T, D);
  GdnWs w{};
  w.t = 0;
  w.g = up(bh * nchunks * CH * CH * 2);
  w.starts = w.g + up(bh * nchunks * CH * 4);
  const size_t seg = P > 1 ? bh * P * (size_t)D * D * 4 : 0;
  w.trans = w.starts + up(seg);
  w.total = w.trans + up(seg);
  return w;
}
}  // namespace

size_t gdn_chunk_workspace(int B, int T, int H, int D) { return gdn_ws_layout(B, T, H, D).total; }

template <int D, int NW, bool OUT>
static hipError_t launch_scan(const GdnScanArgs& a, hipStream_t stream) {
  const long nblk = (long)a.B * a.H * scan_tiles_per_bh(a.nseg_launch, a.tiles, D / (16 * NW));
  if (nblk > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (nblk == 0) return hipSuccess;
  gdn_scan_kernel<D, NW, OUT><<<(unsigned)nblk, 128 * NW, 0, stream>>>(a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_scan_nw(const GdnScanArgs& a, int nw, hipStream_t stream) {
  if (nw == 4) return launch_scan<D, 4, true>(a, stream);
  if (nw == 2) return launch_scan<D, 2, true>(a, stream);
  if (nw == 1) return launch_scan<D, 1, true>(a, stream);
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t launch_scan_segmented(GdnScanArgs a, int P, float* starts, float* trans,
                                        hipStream_t stream) {
  constexpr int NT4 = D / 64;
  const int nchunks = a.nchunks;
  a.seg_chunks = (nchunks + P - 1) / P;
  a.nsegs = P;
  // pass 1: segments 0 .. P-2 without outputs; segment ends -> starts[j + 1],
  // transitions -> trans[j]
  GdnScanArgs p1 = a;
  p1.out = nullptr;
  p1.state_out = nullptr;
  p1.init_seg = nullptr;
  p1.fin_seg = starts;
  p1.fin_trans = trans;
  p1.nseg_launch = P - 1;
  p1.tiles = 2 * NT4;
  hipError_t e = launch_scan<D, 4, false>(p1, stream);
  if (e != hipSuccess) return e;
  gdn_seg_combine_kernel<D><<<(unsigned)(a.B * a.H * (D / 16)), 512, 0, stream>>>(a.state_in, starts, trans, P);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // pass 2: all segments from their true starts, with outputs
  GdnScanArgs p2 = a;
  p2.init_seg = starts;
  p2.fin_seg = nullptr;
  p2.fin_trans = nullptr;
  p2.nseg_launch = P;
  p2.tiles = NT4;
  return launch_scan<D, 4, true>(p2, stream);
}

hipError_t launch_gdn_chunk(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const float* alpha, const float* beta, const float* state_in,
                            uint16_t* out, float* state_out, int B, int T, int H, int D, int nw,
                            void* workspace, hipStream_t stream, hipEvent_t after_prep) {
  if (D != 64 && D != 128) return hipErrorInvalidValue;
  const int nchunks = (T + CH - 1) / CH;
  const size_t nt = (size_t)B * H * nchunks;
  const GdnWs w = gdn_ws_layout(B, T, H, D);
  uint8_t* wsb = reinterpret_cast<uint8_t*>(workspace);
  uint16_t* t_ws = reinterpret_cast<uint16_t*>(wsb + w.t);
  float* g_ws = reinterpret_cast<float*>(wsb + w.g);
  if (nchunks > 0) {
    if (nt > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (D == 128) gdn_prep_kernel<128><<<(unsigned)nt, 64, 0, stream>>>(k, alpha, beta, t_ws, g_ws, T, H, nchunks);
    else gdn_prep_kernel<64><<<(unsigned)nt, 64, 0, stream>>>(k, alpha, beta, t_ws, g_ws, T, H, nchunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (after_prep) {
    const hipError_t e = hipEventRecord(after_prep, stream);
    if (e != hipSuccess) return e;
  }
  GdnScanArgs a;
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.t_in = t_ws; a.g_in = g_ws; a.out = out;
  a.state_in = state_in; a.state_out = state_out;
  a.init_seg = nullptr; a.fin_seg = nullptr; a.fin_trans = nullptr;
  a.B = B; a.T = T; a.H = H; a.nchunks = nchunks;
  a.seg_chunks = nchunks; a.nsegs = 1; a.nseg_launch = 1;
  const int P = gdn_segments(B, H, T, D);
  if (P > 1) {
    float* starts = reinterpret_cast<float*>(wsb + w.starts);
    float* trans = reinterpret_cast<float*>(wsb + w.trans);
    return D == 128 ? launch_scan_segmented<128>(a, P, starts, trans, stream)
                    : launch_scan_segmented<64>(a, P, starts, trans, stream);
  }
  if (nw <= 0) nw = gdn_chunk_waves(B, H, D);
  a.tiles = D / (16 * nw);
  return D == 128 ? launch_scan_nw<128>(a, nw, stream) : launch_scan_nw<64>(a, nw, stream);
}

}  // namespace kairos
