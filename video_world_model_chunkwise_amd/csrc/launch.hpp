// Host-callable launchers of the gfx950 kernels (one per kernel family).
// Every launcher only enqueues work on `stream` and returns the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kairos {

// Arguments of the windowed-attention kernel (SWA / DSWA / hybrid epilogue).
struct WinArgs {
  const void* q;            // bf16 [B][T][H][128] or E4M3 codes
  const void* k;            // same type as q
  const uint16_t* v;        // bf16 [B][T][H][128]
  const float* q_scales;    // [B][H][nblk] (FP8 only)
  const float* k_scales;
  // second (DSWA) branch of the hybrid kernel: its own q, k (and scales) when
  // they differ from the first branch's (RoPE at the group positions); null
  // means the first branch's
  const void* q2;
  const void* k2;
  const float* q_scales2;
  const float* k_scales2;
  const uint16_t* k_ring;   // [B][R][L][H][128] bf16 or null
  const uint16_t* k_ring2;  // keys of the second branch's ring frames when they differ
                            // from the first branch's (RoPE at the group positions)
  const uint16_t* v_ring;
  const uint16_t* o_gdn;    // bf16 [B][T][H][128] (hybrid only); null: the epilogue leaves
                            // sig(z_swa) o_swa + sig(z_dswa) o_dswa (fp32) in ypart and
                            // launch_hlta_combine adds the gated GDN branch
  const float* gates;       // logits [3][H] (hybrid only)
  float* ypart;             // fp32 [B][T][H][128] scratch for the first branch (hybrid only)
  float* ylse;              // fp32 [B][T][H] scratch: log-sum-exp of a parked partial result (hybrid only)
  uint16_t* out;            // bf16 [B][T][H][128]
  int B, T, H, L, F, QT;    // F frames in the call (last may be partial), QT query tiles per frame
  int w, dil, R, nblk;
  int centered;             // 0: causal window (i - w, i]; 1: centred |j - i| <= w / 2
  // quantisation blocks of FP8 / FP4 Q and K: nbf == 0 -> 64-token blocks in
  // the call's token order (scale of token t at t / 64); nbf > 0 -> blocks
  // restart at every frame (scale of row m of call frame f at f * nbf + m / 64,
  // and of a ring frame in slot s at s * nbf + m / 64 of ks_ring [B][H][R][nbf])
  int nbf;
  const float* ks_ring;     // key scales of the ring frames (quantised keys in a ring)
  const float* ks_ring2;    // the same for the second branch's own keys
  long frame_offset;
};

// Arguments of the gated-delta-rule input prologue (one row = one (token, head)).
struct PrologueArgs {
  const void* k_in;         // [rows][D] io type
  const void* q_in;         // [rows][D] or null (query not normalised)
  const void* v_in;         // [rows][D] or null (canonical form)
  const float* za;          // [rows] decay logits
  const float* zb;          // [rows] write-strength logits
  void* k_out;
  void* q_out;
  void* v_out;
  float* alpha;             // [rows]
  float* beta;              // [rows]
  long rows;
};

// Windowed-branch operands: E4M3 quantisation and/or RoPE of q and/or k
// ([B][T][H][D] bf16) at a branch's positions (frame_offset, L, dil), written
// as bf16 or as E4M3 codes with per-(b, h, 64-token block) scales.
struct OperandArgs {
  const uint16_t* x[2];     // nt tensors sharing positions (q and k of one branch)
  void* out[2];
  float* scales[2];         // FP8 only: [B][H][nblk]
  int nt, B, T, H, L, dil, nblk;
  int nbf;                  // 0: 64-token blocks in the call's token order; > 0: blocks restart
                            // at every frame, nbf = ceil(L / 64) per frame (nblk = frames * nbf)
  long frame_offset;
};
struct RopeFreqs {
  double theta[64];         // base^(-2i/D), i < D/2
};
// fmt: 0 bf16 out, 1 E4M3 codes, 2 E2M1 codes (two per byte)
hipError_t launch_rope(const OperandArgs& args, int D, double base, int fmt, hipStream_t stream);

// fp32 io when f32, else bf16; D in {32, 64, 128}
hipError_t launch_gdn_prologue(const PrologueArgs& args, int D, bool f32, bool normalize_q,
                               bool literal, hipStream_t stream);

hipError_t launch_gdn_f32(const float* q, const float* k, const float* v, const float* alpha,
                          const float* beta, const float* state_in, float* out, float* state_out,
                          int B, int T, int H, int D, hipStream_t stream);
// Chunkwise bf16 gated delta rule: a parallel per-chunk prep kernel (decays,
// T = (I + A)^{-1}) into `workspace` (gdn_chunk_workspace bytes), then the
// sequential scan, split over time into gdn_segments() segments when there
// are few (b, h) (two scan passes and a combine).  nw: waves per scan
// workgroup of the unsplit scan (16 nw rows of S per workgroup); <= 0 picks
// by problem size.
hipError_t launch_gdn_chunk(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const float* alpha, const float* beta, const float* state_in,
                            uint16_t* out, float* state_out, int B, int T, int H, int D, int nw,
                            void* workspace, hipStream_t stream,
                            hipEvent_t after_prep = nullptr);
int gdn_chunk_waves(int B, int H, int D);
size_t gdn_chunk_workspace(int B, int T, int H, int D);
int gdn_segments(int B, int H, int T, int D);
// Block quantiser: fmt 1 E4M3 (codes [B][T][H][D] bytes), 2 E2M1 (codes
// [B][T][H][D/2] bytes); scales [B][H][ceil(T/64)]
hipError_t launch_block_quant(const uint16_t* x, uint8_t* codes, float* scales, int B, int T, int H,
                              int D, int fmt, hipStream_t stream, int L = 1, int nbf = 0);
// Ring update of a streamed call: copy the call's last min(R, F) frames of
// src ([B][F * L][H][row_bytes]) into ring slots (frame_offset + f) mod R of
// dst ([B][R][L][H][row_bytes]).
hipError_t launch_ring_copy(const void* src, void* dst, int B, int F, int L, int H, int row_bytes,
                            long frame_offset, int R, hipStream_t stream);
// The same for per-frame key scales: src [BH][F][nbf] fp32 -> dst [BH][R][nbf].
hipError_t launch_ring_copy_scales(const float* src, float* dst, int BH, int F, int nbf, long frame_offset,
                                   int R, hipStream_t stream);
// qf: 0 bf16 q, k; 1 E4M3 codes; 2 E2M1 codes (two per byte)
hipError_t launch_window(const WinArgs& args, int qf, bool hybrid, hipStream_t stream);
// Workgroups of one window-kernel launch over B x T x H with frames of L tokens.
long window_workgroups(int B, int T, int H, int L);

// y = bf16_rne(ypart + sig(z_gdn[h]) o_gdn) over [B][T][H][128] (the hybrid
// window kernel's epilogue when the GDN branch ran beside it).
hipError_t launch_hlta_combine(const float* ypart, const uint16_t* o_gdn, const float* gates,
                               uint16_t* out, int B, int T, int H, hipStream_t stream);

}  // namespace kairos
