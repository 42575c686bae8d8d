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
