// Key/value ring update of a streamed rollout.
//
// Ring (Kairos paper, Sec. 2.2.2 "Long-Horizon Generation": constant memory
// per step through recurrent state passing): a streamed call keeps the last R
// frames of K and V in slots f mod R; the update copies the call's last
// min(R, F) frames into their slots after the call's attention has read the
// ring.
#include "common.hpp"
#include "launch.hpp"

namespace kairos {

// Copy frames [f_first, F) of the call ([B][F*L][row]) into ring slots
// (frame_offset + f) mod R of [B][R][L][row], 16-byte granules.
__global__ __launch_bounds__(256) void ring_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        long frame16, int T_frames, int f_first,
                                                        long frame_offset, int R) {
  const int fi = blockIdx.y;                      // 0 .. nframes-1
  const int b = blockIdx.z;
  const int f = f_first + fi;
  const int slot = (int)((frame_offset + f) % R);
  const uint4* s = src + ((size_t)b * T_frames + f) * frame16;
  uint4* d = dst + ((size_t)b * R + slot) * frame16;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < frame16; i += (long)gridDim.x * 256) d[i] = s[i];
}

hipError_t launch_ring_copy(const void* src, void* dst, int B, int F, int L, int H, int row_bytes,
                            long frame_offset, int R, hipStream_t stream) {
  const int n = F < R ? F : R;
  if (n <= 0) return hipSuccess;
  const long frame16 = (long)L * H * row_bytes / 16;
  dim3 grid((unsigned)((frame16 + 255) / 256 < 1024 ? (frame16 + 255) / 256 : 1024), n, B);
  ring_copy_kernel<<<grid, 256, 0, stream>>>(reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst),
                                             frame16, F, F - n, frame_offset, R);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void ring_copy_scales_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                               int BH, int F, int f_first, int nbf, long frame_offset,
                                                               int R) {
  const long n = (long)BH * (F - f_first) * nbf;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const long bh = i / ((long)(F - f_first) * nbf);
    const int rest = (int)(i % ((long)(F - f_first) * nbf));
    const int f = f_first + rest / nbf, j = rest % nbf;
    const int slot = (int)((frame_offset + f) % R);
    dst[(bh * R + slot) * nbf + j] = src[(bh * F + f) * nbf + j];
  }
}

hipError_t launch_ring_copy_scales(const float* src, float* dst, int BH, int F, int nbf, long frame_offset,
                                   int R, hipStream_t stream) {
  const int n = F < R ? F : R;
  if (n <= 0 || nbf <= 0) return hipSuccess;
  const long total = (long)BH * n * nbf;
  const long nb = (total + 255) / 256;
  ring_copy_scales_kernel<<<(unsigned)(nb < 4096 ? nb : 4096), 256, 0, stream>>>(src, dst, BH, F, F - n, nbf,
                                                                                 frame_offset, R);
  return hipGetLastError();
}

}  // namespace kairos
