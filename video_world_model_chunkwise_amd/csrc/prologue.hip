// Input prologue of the gated delta rule, one pass over the per-token inputs:
//   k_hat = k / ||k||_2 per (token, head) row (Kairos paper, Sec. 2.2.1,
//           Eq. 2-3: the delta-rule write and retrieval take unit keys);
//   q_hat = q / ||q||_2 (optional);
//   alpha = sigma(z_alpha)                     (Eq. 4)
//   beta  = sigma(z_beta)                      (Eq. 1)
// and, for the printed Eq. 6 (erase with the un-decayed retrieval), the
// rescaled inputs under which the canonical recurrence equals it:
//   beta' = beta / alpha = (1 + e^{-z_alpha}) / (1 + e^{-z_beta}),  v' = alpha v.
// A zero row stays zero.  The norm is taken after an exact power-of-two
// rescaling of the row by its largest magnitude, so rows whose squares would
// under- or overflow in fp32 still normalise.
//
// Memory-bound: every byte is read and written once.  A row of d elements is
// d * esz / 16 lanes, one 16-byte vector each; a wave covers consecutive
// rows, so each load or store instruction moves one contiguous 1 KiB span.
// Every lane issues all its loads (U = 2 rows per tensor) before their first
// use; deeper unrolling (U = 4, 8) measured slower.
#include "common.hpp"
#include "launch.hpp"

namespace kairos {

namespace {

// 16 bytes of one io type <-> fp32 values
template <typename E> struct Lane16;

template <> struct Lane16<uint16_t> {          // bf16
  static constexpr int N = 8;
  __device__ static void unpack(uint4 u, float* f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = __uint_as_float(w[e] << 16);
      f[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
  __device__ static uint4 pack(const float* f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
  }
};

template <> struct Lane16<float> {
  static constexpr int N = 4;
  __device__ static void unpack(uint4 u, float* f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
  __device__ static uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};

// reductions over aligned groups of W lanes (every lane of the wave takes part)
template <int W>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
  for (int m = W / 2; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, W));
  return x;
}

template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = W / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, W);
  return x;
}

// Normalise one row held as W lanes x N values.
template <int W, int N>
__device__ __forceinline__ void normalize_row(float* f) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) m = fmaxf(m, fabsf(f[i]));
  m = group_max<W>(m);
  int e;
  (void)frexpf(m, &e);                 // m = mant * 2^e, mant in [0.5, 1); e = 0 for m = 0
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    f[i] = ldexpf(f[i], -e);           // exact; the row's largest magnitude is now in [0.5, 1)
    ss = fmaf(f[i], f[i], ss);
  }
  ss = group_sum<W>(ss);
  const float r = m > 0.f ? 1.0f / sqrtf(ss) : 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) f[i] *= r;
}

// Streaming accesses: every byte is touched once, so loads and stores are
// marked non-temporal (measured 3-9% faster than plain ones at B4 T57600 H24).
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load16(const void* base, long off_bytes, bool ok) {
  if (!ok) return make_uint4(0u, 0u, 0u, 0u);
  const nt_u32x4 t = __builtin_nontemporal_load(
      reinterpret_cast<const nt_u32x4*>(reinterpret_cast<const uint8_t*>(base) + off_bytes));
  return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ void store16(void* base, long off_bytes, uint4 v) {
  const nt_u32x4 t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<nt_u32x4*>(reinterpret_cast<uint8_t*>(base) + off_bytes));
}

constexpr int kPrologueThreads = 256;
constexpr int kPrologueRowsPerLane = 2;

template <typename E, int D>
struct PrologueGeom {
  static constexpr int N = Lane16<E>::N;          // values per lane
  static constexpr int LPR = D / N;               // lanes per row
  static constexpr int RPW = 64 / LPR;            // rows per wave and pass
  static constexpr int U = kPrologueRowsPerLane;  // passes per wave
  static constexpr int RPB = (kPrologueThreads / 64) * U * RPW;  // rows per workgroup
};

}  // namespace

// Inputs and outputs may coincide exactly (in place): each lane reads all its
// bytes before it writes any of them, and no other lane touches them.
template <typename E, int D, bool NQ, bool LIT>
__global__ __launch_bounds__(kPrologueThreads) void gdn_prologue_kernel(PrologueArgs a) {
  using G = PrologueGeom<E, D>;
  using P = Lane16<E>;
  constexpr int N = G::N, LPR = G::LPR, RPW = G::RPW, U = G::U;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPR;
  const long row0 = (long)blockIdx.x * G::RPB + (long)wave * U * RPW + lane / LPR;
  const long col_bytes = (long)sub * 16;

  uint4 kv[U], qv[U], vv[U];
  float za[U], zb[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const long row = row0 + (long)u * RPW;
    const bool ok = row < a.rows;
    const long off = row * (long)(D * sizeof(E)) + col_bytes;
    kv[u] = load16(a.k_in, off, ok);
    if (NQ) qv[u] = load16(a.q_in, off, ok);
    if (LIT) vv[u] = load16(a.v_in, off, ok);
    za[u] = ok ? a.za[row] : 0.f;
    zb[u] = ok ? a.zb[row] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const long row = row0 + (long)u * RPW;
    const bool ok = row < a.rows;
    const long off = row * (long)(D * sizeof(E)) + col_bytes;
    float f[N];
    P::unpack(kv[u], f);
    normalize_row<LPR, N>(f);
    if (ok) store16(a.k_out, off, P::pack(f));
    if (NQ) {
      P::unpack(qv[u], f);
      normalize_row<LPR, N>(f);
      if (ok) store16(a.q_out, off, P::pack(f));
    }
    const float ea = expf(-za[u]), eb = expf(-zb[u]);
    const float alpha = 1.0f / (1.0f + ea);
    const float beta = LIT ? (1.0f + ea) / (1.0f + eb) : 1.0f / (1.0f + eb);
    if (LIT) {
      P::unpack(vv[u], f);
#pragma unroll
      for (int i = 0; i < N; ++i) f[i] *= alpha;
      if (ok) store16(a.v_out, off, P::pack(f));
    }
    if (ok && sub == 0) {
      a.alpha[row] = alpha;
      a.beta[row] = beta;
    }
  }
}

namespace {

template <typename E, int D>
hipError_t launch_prologue_d(const PrologueArgs& a, bool nq, bool lit, hipStream_t s) {
  using G = PrologueGeom<E, D>;
  const long blocks = (a.rows + G::RPB - 1) / G::RPB;
  const dim3 grid((unsigned)blocks), block(kPrologueThreads);
  if (nq && lit) gdn_prologue_kernel<E, D, true, true><<<grid, block, 0, s>>>(a);
  else if (nq) gdn_prologue_kernel<E, D, true, false><<<grid, block, 0, s>>>(a);
  else if (lit) gdn_prologue_kernel<E, D, false, true><<<grid, block, 0, s>>>(a);
  else gdn_prologue_kernel<E, D, false, false><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_prologue_e(const PrologueArgs& a, int D, bool nq, bool lit, hipStream_t s) {
  switch (D) {
    case 32: return launch_prologue_d<E, 32>(a, nq, lit, s);
    case 64: return launch_prologue_d<E, 64>(a, nq, lit, s);
    case 128: return launch_prologue_d<E, 128>(a, nq, lit, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gdn_prologue(const PrologueArgs& a, int D, bool f32, bool normalize_q,
                               bool literal, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  return f32 ? launch_prologue_e<float>(a, D, normalize_q, literal, stream)
             : launch_prologue_e<uint16_t>(a, D, normalize_q, literal, stream);
}

}  // namespace kairos
