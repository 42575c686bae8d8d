// Operands of the windowed branches: the FP8 E4M3 and the 4-bit (FP4 E2M1)
// block quantisers of Q and K, RoPE of Q and K, and RoPE fused with either.
//
// Quantisation (Kairos project page, Sec. 2 Q2: FP8/INT4 attention quantisation;
// block size and scale rule as in the 64-token-block absmax workload): per
// (b, h, 64 consecutive tokens, all d): s = amax / 448 in fp32 (1 when
// amax == 0); code = E4M3(x / s) of the correctly rounded fp32 quotient,
// round to nearest even, saturating at 448.
//
// The quotient is x * r with r = RN(1/s) (one division per wave), corrected
// by one residual step: e = fma(-q, s, x) is exact and fma(e, r, q) is the
// correctly rounded x / s (Markstein's theorem for a reciprocal within half
// an ulp and a first quotient within one ulp; no under- or overflow can
// change a code here: |x / s| <= 448 and quotients below 2^-126 encode as
// zero).  The sign of a zero quotient is taken from x.  The encoding is the
// gfx950 conversion instruction (OCP E4M3, round to nearest even) on values
// first clamped to +-448, so its saturation mode never matters.
//
// 4-bit codes (OCP FP4 E2M1: sign, 2 exponent bits with bias 1, 1 mantissa
// bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6): s = amax / 6, the same
// correctly rounded quotient clamped to +-6, rounded to the nearest code with
// each tie (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) going to the code with
// mantissa bit 0 (the gfx950 conversion instruction); feature 2i is the low
// nibble of byte i.
//
// RoPE (Kairos paper, arXiv 2606.16533 HTML v3, Sec. 2.2.2: every
// sliding-window attention block uses RoPE-based relative positional
// encoding).  The variant is RoFormer's (Su et al., Eq. 13-15): feature pairs
// (2i, 2i+1) of a token at position p are rotated by p * theta_i, theta_i =
// base^(-2i/d).  A branch's positions are those of the sequence it attends
// over: p = (f div dil) * L + (t mod L), f the absolute frame index (SWA: the
// absolute token index; DSWA: the position in the residue group's
// sub-sequence of Eq. 8).  With FP8 the rotated fp32 values are quantised.
//
// Work decomposition (memory-bound: every byte moves once): one wave per
// (b, head, 64-token block).  A token row of d bf16 is d/8 lanes of 16 bytes,
// so each load instruction of a wave covers 512/d consecutive tokens' rows
// and the wave issues its whole 64-token block (16 KB at d = 128) before the
// first use.  The block maximum is a wave reduction (no barrier).  The four
// waves of a workgroup take four adjacent heads of the same token block (rows
// adjacent in memory); with RoPE they share the block's cos/sin table in LDS
// (angle in fp64, reduced to [-pi, pi], then fp32 sincos), and q and k of a
// branch, which share positions, are done by the same workgroup.
#include "common.hpp"
#include "launch.hpp"

namespace kairos {

namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;
constexpr double kInvTwoPi = 0.15915494309189533576888376337251;

template <int D>
struct OperandGeom {
  static constexpr int LPR = D / 8;          // lanes per token row
  static constexpr int TPI = 64 / LPR;       // tokens per load instruction
  static constexpr int NI = 64 / TPI;        // load instructions per 64-token block
  static constexpr int NP = D / 2;           // RoPE frequencies
  static constexpr int CST = NP + 2;         // cos/sin table row stride (float2), 16-byte aligned
};

// fp32 values of one lane's 8 features (token row of load i); with RoPE the
// features' 4 pairs are rotated by the table row of that token.
template <int D, bool ROPE>
__device__ __forceinline__ void operand_values(uint4 v, const float2* csrow, float* y) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x0 = __uint_as_float(w[e] << 16), x1 = __uint_as_float(w[e] & 0xFFFF0000u);
    if (ROPE) {
      const float2 c = csrow[e];
      y[2 * e] = x0 * c.x - x1 * c.y;
      y[2 * e + 1] = x0 * c.y + x1 * c.x;
    } else {
      y[2 * e] = x0;
      y[2 * e + 1] = x1;
    }
  }
}

// Correctly rounded y / s from r = RN(1 / s) (one residual step), sign of
// zero from y.
__device__ __forceinline__ float quotient(float y, float s, float r) {
  const float t = y * r;
  return copysignf(fmaf(fmaf(-t, s, y), r, t), y);
}

// E2M1 codes of y[0..7] / s, two per byte (element 2i in the low nibble):
// the gfx950 conversion instruction (scale 1) on the quotients clamped to
// +-6.  On clamped inputs it rounds exactly as counting the rounding
// thresholds does (nearest, ties to the even code, sign of zero kept):
// checked on every bf16 value of magnitude <= 8 and every tie +-1 ulp.
__device__ __forceinline__ uint32_t e2m1_encode8(const float* y, float s, float r) {
  float q[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) q[e] = __builtin_amdgcn_fmed3f(quotient(y[e], s, r), -6.f, 6.f);
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q[0], q[1], 1.f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[2], q[3], 1.f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[4], q[5], 1.f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[6], q[7], 1.f, 3);
  return w;
}

// E4M3 codes of y[0..7] / s (bytes in order), r = RN(1 / s).
__device__ __forceinline__ uint2 e4m3_encode8(const float* y, float s, float r) {
  float q[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) q[e] = __builtin_amdgcn_fmed3f(quotient(y[e], s, r), -448.f, 448.f);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], hi, true);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

}  // namespace

// OUT: 0 bf16, 1 E4M3 codes, 2 E2M1 codes (packed two per byte)
template <int D, bool ROPE, int OUT>
__global__ __launch_bounds__(256) void qk_operand_kernel(OperandArgs a, RopeFreqs fr) {
  constexpr bool FP8 = OUT != 0;               // quantised: block scales
  constexpr float QMAX = OUT == 2 ? 6.f : 448.f;
  using G = OperandGeom<D>;
  constexpr int LPR = G::LPR, TPI = G::TPI, NI = G::NI, NP = G::NP, CST = G::CST;
  __shared__ __attribute__((aligned(16))) float2 cs[ROPE ? 64 * CST : 2];
  const int blk = blockIdx.x, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = 4 * blockIdx.y + wave;
  // the block's first token and its number of tokens: 64 in token order, or
  // (frame-aligned blocks) up to the end of the block's frame
  int t0, tn;
  if (a.nbf > 0) {
    const int fb = blk / a.nbf, ib = blk % a.nbf;
    t0 = fb * a.L + 64 * ib;
    tn = min(64, min(a.L - 64 * ib, a.T - t0));
  } else {
    t0 = blk * 64;
    tn = min(64, a.T - t0);
  }

  if (ROPE) {
    for (int e = threadIdx.x; e < 64 * NP; e += 256) {
      const int tl = e / NP, i = e % NP;
      const int t = t0 + min(tl, tn - 1);
      const long f = a.frame_offset + t / a.L;
      const long p = (f / a.dil) * a.L + t % a.L;
      const double ang = (double)p * fr.theta[i];
      const double r = ang - rint(ang * kInvTwoPi) * kTwoPi;      // |r| <= pi
      float sn, cn;
      sincosf((float)r, &sn, &cn);
      cs[tl * CST + i] = make_float2(cn, sn);
    }
    __syncthreads();
  }
  if (h >= a.H) return;

  const int sub = lane % LPR, tsub = lane / LPR;
  for (int n = 0; n < a.nt; ++n) {
    uint4 v[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int tl = i * TPI + tsub, t = t0 + tl;
      v[i] = tl < tn ? *reinterpret_cast<const uint4*>(a.x[n] + (((size_t)b * a.T + t) * a.H + h) * D + 8 * sub)
                     : make_uint4(0u, 0u, 0u, 0u);
    }
    auto csrow = [&](int i) { return cs + (i * TPI + tsub) * CST + 4 * sub; };
    if (OUT == 0) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int tl = i * TPI + tsub, t = t0 + tl;
        float y[8];
        operand_values<D, ROPE>(v[i], ROPE ? csrow(i) : nullptr, y);
        if (tl < tn)
          *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out[n]) + (((size_t)b * a.T + t) * a.H + h) * D + 8 * sub) =
              make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                         pack_bf16x2(y[6], y[7]));
      }
    } else {
      float amax = 0.f;                      // rows past the block are zero
      if (ROPE) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          float y[8];
          operand_values<D, ROPE>(v[i], csrow(i), y);
#pragma unroll
          for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[e]));
        }
        // the table is read again below: the rotations are recomputed rather
        // than kept live (128 values per lane) across the reduction
        asm volatile("" ::: "memory");
      } else {
        // magnitude order of finite bf16 values is the integer order of their
        // low 15 bits: the block maximum needs no conversion
        uint32_t mbits = 0;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) mbits = max(mbits, max(w[e] & 0x7FFFu, (w[e] >> 16) & 0x7FFFu));
        }
        amax = __uint_as_float(mbits << 16);
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
      const float s = amax > 0.f ? amax / QMAX : 1.f;
      const float r = 1.f / s;
      if (lane == 0) a.scales[n][((size_t)b * a.H + h) * a.nblk + blk] = s;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int tl = i * TPI + tsub, t = t0 + tl;
        float y[8];
        operand_values<D, ROPE>(v[i], ROPE ? csrow(i) : nullptr, y);
        if (OUT == 1) {
          const uint2 c = e4m3_encode8(y, s, r);
          if (tl < tn)
            *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(a.out[n]) + (((size_t)b * a.T + t) * a.H + h) * D + 8 * sub) = c;
        } else {
          const uint32_t c = e2m1_encode8(y, s, r);
          if (tl < tn)
            *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(a.out[n]) + ((((size_t)b * a.T + t) * a.H + h) * D + 8 * sub) / 2) = c;
        }
      }
    }
  }
}

namespace {

template <int D, bool ROPE, int OUT>
void launch_operands_t(const OperandArgs& a, const RopeFreqs& fr, hipStream_t s) {
  const dim3 grid((unsigned)a.nblk, (unsigned)((a.H + 3) / 4), (unsigned)a.B);
  qk_operand_kernel<D, ROPE, OUT><<<grid, 256, 0, s>>>(a, fr);
}

template <bool ROPE, int OUT>
hipError_t launch_operands(const OperandArgs& a, int D, const RopeFreqs& fr, hipStream_t s) {
  switch (D) {
    case 32: launch_operands_t<32, ROPE, OUT>(a, fr, s); break;
    case 64: launch_operands_t<64, ROPE, OUT>(a, fr, s); break;
    case 128: launch_operands_t<128, ROPE, OUT>(a, fr, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_quant(const uint16_t* x, uint8_t* codes, float* scales, int B, int T, int H,
                              int D, int fmt, hipStream_t stream, int L, int nbf) {
  if (T <= 0) return hipSuccess;
  OperandArgs a{};
  a.x[0] = x;
  a.out[0] = codes;
  a.scales[0] = scales;
  a.nt = 1;
  a.B = B;
  a.T = T;
  a.H = H;
  a.L = L > 0 ? L : 1;
  a.dil = 1;
  a.nbf = nbf;
  a.nblk = nbf > 0 ? ((T + a.L - 1) / a.L) * nbf : (T + 63) / 64;
  RopeFreqs fr{};
  return fmt == 2 ? launch_operands<false, 2>(a, D, fr, stream) : launch_operands<false, 1>(a, D, fr, stream);
}

hipError_t launch_rope(const OperandArgs& a, int D, double base, int fmt, hipStream_t stream) {
  if (a.T <= 0 || a.nt <= 0) return hipSuccess;
  RopeFreqs fr;
  for (int i = 0; i < 64; ++i) fr.theta[i] = i < D / 2 ? pow(base, -2.0 * i / D) : 0.0;
  switch (fmt) {
    case 0: return launch_operands<true, 0>(a, D, fr, stream);
    case 1: return launch_operands<true, 1>(a, D, fr, stream);
    case 2: return launch_operands<true, 2>(a, D, fr, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kairos
