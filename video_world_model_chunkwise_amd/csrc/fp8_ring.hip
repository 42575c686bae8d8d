// FP8 E4M3 quantisation of the windowed branches' Q and K, and the
// key/value ring update of a streamed rollout.
//
// Quantisation (Kairos project page, TL;DR / Q3: FP8 attention quantisation;
// block size and scale rule as in the 64-token-block absmax workload): per
// (b, h, 64 consecutive tokens, all d): s = amax / 448 in fp32 (1 when
// amax == 0); code = E4M3(x / s) with an IEEE fp32 division, round to
// nearest even, saturating at 448.  OCP E4M3: 1 sign, 4 exponent (bias 7),
// 3 mantissa bits, subnormals down to 2^-9, no infinities.  The conversion is
// done with integer arithmetic on the fp32 bit pattern, so it does not depend
// on any conversion instruction's saturation mode.
//
// Ring (Kairos paper, Sec. 2.2.2 "Long-Horizon Generation": constant memory
// per step through recurrent state passing): a streamed call keeps the last R
// frames of K and V in slots f mod R; the update copies the call's last
// min(R, F) frames into their slots after the call's attention has read the
// ring.
#include "common.hpp"
#include "launch.hpp"

namespace kairos {

__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t code;
  if (!(a < 448.f)) {
    code = 0x7Eu;                                   // saturate (inputs are finite)
  } else if (a < 0.015625f) {                       // below 2^-6: subnormal grid 2^-9
    code = (uint32_t)rintf(a * 512.f);              // exact scaling; rint = ties to even
  } else {
    const uint32_t au = __float_as_uint(a);
    int e = (int)(au >> 23) - 127;                  // -6 .. 8
    uint32_t m = au & 0x7FFFFFu;
    uint32_t r = m >> 20;                           // top 3 mantissa bits
    const uint32_t rem = m & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
    if (r == 8u) { r = 0u; ++e; }
    code = ((uint32_t)(e + 7) << 3) | r;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

template <int D>
__global__ __launch_bounds__(256) void fp8_quant_kernel(const uint16_t* __restrict__ x,
                                                        uint8_t* __restrict__ codes,
                                                        float* __restrict__ scales, int T, int H,
                                                        int nblk) {
  constexpr int TPT = D / 32;             // threads per token (32 features each)
  constexpr int TOK = 256 / TPT;          // tokens covered per pass
  constexpr int PASSES = TOK >= 64 ? 1 : 64 / TOK;
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int part = tid % TPT;
  __shared__ float red[4];
  uint4 vals[PASSES][4];
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int tl = p * TOK + tid / TPT;
    const int t = blk * 64 + tl;
#pragma unroll
    for (int j = 0; j < 4; ++j) vals[p][j] = make_uint4(0, 0, 0, 0);
    if (tl < 64 && t < T) {
      const uint4* src = reinterpret_cast<const uint4*>(x + (((size_t)b * T + t) * H + h) * D + 32 * part);
#pragma unroll
      for (int j = 0; j < 4; ++j) vals[p][j] = src[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w[4] = {vals[p][j].x, vals[p][j].y, vals[p][j].z, vals[p][j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        amax = fmaxf(amax, fabsf(__uint_as_float(w[e] << 16)));
        amax = fmaxf(amax, fabsf(__uint_as_float(w[e] & 0xFFFF0000u)));
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if (tid % 64 == 0) red[tid / 64] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax > 0.f ? amax / 448.f : 1.f;
  if (tid == 0) scales[((size_t)b * H + h) * nblk + blk] = s;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int tl = p * TOK + tid / TPT;
    const int t = blk * 64 + tl;
    if (tl >= 64 || t >= T) continue;
    uint32_t outw[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w[4] = {vals[p][j].x, vals[p][j].y, vals[p][j].z, vals[p][j].w};
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const uint32_t c0 = e4m3_code(__uint_as_float(w[e] << 16) / s);
        const uint32_t c1 = e4m3_code(__uint_as_float(w[e] & 0xFFFF0000u) / s);
        const uint32_t c2 = e4m3_code(__uint_as_float(w[e + 1] << 16) / s);
        const uint32_t c3 = e4m3_code(__uint_as_float(w[e + 1] & 0xFFFF0000u) / s);
        outw[2 * j + e / 2] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
      }
    }
    uint4* dst = reinterpret_cast<uint4*>(codes + (((size_t)b * T + t) * H + h) * D + 32 * part);
    dst[0] = make_uint4(outw[0], outw[1], outw[2], outw[3]);
    dst[1] = make_uint4(outw[4], outw[5], outw[6], outw[7]);
  }
}

hipError_t launch_fp8_quant(const uint16_t* x, uint8_t* codes, float* scales, int B, int T, int H,
                            int D, hipStream_t stream) {
  const int nblk = (T + 63) / 64;
  if (nblk == 0) return hipSuccess;
  dim3 grid(nblk, H, B);
  switch (D) {
    case 32: fp8_quant_kernel<32><<<grid, 256, 0, stream>>>(x, codes, scales, T, H, nblk); break;
    case 64: fp8_quant_kernel<64><<<grid, 256, 0, stream>>>(x, codes, scales, T, H, nblk); break;
    case 128: fp8_quant_kernel<128><<<grid, 256, 0, stream>>>(x, codes, scales, T, H, nblk); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Copy frames [f_first, F) of the call (K and V, [B][F*L][H][D]) into ring
// slots (frame_offset + f) mod R of [B][R][L][H][D].  16-byte granules.
__global__ __launch_bounds__(256) void ring_update_kernel(const uint4* __restrict__ k,
                                                          const uint4* __restrict__ v,
                                                          uint4* __restrict__ k_ring,
                                                          uint4* __restrict__ v_ring,
                                                          long frame_elems16, int T_frames,
                                                          int f_first, long frame_offset, int R) {
  const int fi = blockIdx.y;                      // 0 .. nframes-1
  const int b = blockIdx.z;
  const int f = f_first + fi;
  const int slot = (int)((frame_offset + f) % R);
  const uint4* ks = k + ((size_t)b * T_frames + f) * frame_elems16;
  const uint4* vs = v + ((size_t)b * T_frames + f) * frame_elems16;
  uint4* kd = k_ring + ((size_t)b * R + slot) * frame_elems16;
  uint4* vd = v_ring + ((size_t)b * R + slot) * frame_elems16;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < frame_elems16; i += (long)gridDim.x * 256) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

hipError_t launch_ring_update(const uint16_t* k, const uint16_t* v, uint16_t* k_ring,
                              uint16_t* v_ring, int B, int F, int L, int H, int D, long frame_offset,
                              int R, hipStream_t stream) {
  const int n = F < R ? F : R;
  if (n <= 0) return hipSuccess;
  const long elems16 = (long)L * H * D / 8;
  dim3 grid((unsigned)((elems16 + 255) / 256 < 1024 ? (elems16 + 255) / 256 : 1024), n, B);
  ring_update_kernel<<<grid, 256, 0, stream>>>(reinterpret_cast<const uint4*>(k),
                                               reinterpret_cast<const uint4*>(v),
                                               reinterpret_cast<uint4*>(k_ring),
                                               reinterpret_cast<uint4*>(v_ring), elems16, F, F - n,
                                               frame_offset, R);
  return hipGetLastError();
}

}  // namespace kairos
