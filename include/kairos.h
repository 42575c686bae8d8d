/*
 * kairos.h -- C ABI of the MI355X (gfx950) hybrid linear temporal attention
 * forward: the gated delta rule global memory, causal sliding-window and
 * dilated sliding-window softmax attention, per-head sigmoid branch gates,
 * a streaming state carry with a key/value ring, and FP8 E4M3 windowed Q/K.
 *
 * Source of the operations: "Kairos: A Regret-Aware Native World-Action
 * Model Stack for Physical AI" (arXiv 2606.16533, HTML v3):
 *   Sec. 2.2.1, Eq. 1-6 and step 4    gated delta rule, read-out o_t = S_t q_t;
 *                                     its inputs: sigmoid gates (Eq. 1, 4), unit keys
 *   Sec. 2.2.2, Eq. 7                 sliding-window attention, w = L x window_size
 *   Sec. 2.2.2, Eq. 8                 dilated SWA on the frame-rearranged sequence
 *   Sec. 2.2.2, "Long-Horizon Generation"  recurrent state passing, constant memory per step
 * and the project page "Kairos: A Native World Model Stack for Physical AI"
 * (Sec. 2, Q2: FP8/INT4 attention quantisation and a tiled GatedDeltaNet;
 * Sec. 7: the tiled GatedDeltaNet streams its inputs to hide DRAM latency).
 *
 * Conventions shared by every entry point
 * --------------------------------------
 * Layouts (C order, no padding):
 *   q, k, v, out       [B][T][H][d]      (bf16, or fp32 for the fp32 GDN path)
 *   alpha, beta        [B][T][H]         fp32, the gate values themselves
 *   state_in/out       [B][H][dv][dk]    fp32 (the memory S in R^{dv x dk})
 *   gate_logits        [3][H]            fp32, rows (swa, dswa, gdn); sigmoid applied inside
 *   v_ring             [B][R][L][H][d]   bf16, slot s holds absolute frame f with f mod R == s
 *   k_ring             the same for bf16 keys without RoPE; otherwise the layout
 *                      kairos_hlta_ring_size states (rotated keys, codes + scales)
 *   fp8 codes          [B][T][H][d]      uint8 OCP E4M3; scales [B][H][ceil(T/64)] fp32
 * The gated delta rule is the canonical form
 *   S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t,
 * keys arrive L2-normalised (nothing renormalises them).  Windows are causal
 * by default: query i sees keys i-w < j <= i (SWA), or centred on request
 * (|j - i| <= floor(w/2)); DSWA groups frames by absolute frame index mod
 * dilation and applies the same window to positions inside a group.
 * The softmax scale is 1/sqrt(d).
 *
 * Ownership and streams: the caller owns every buffer (device memory unless
 * stated).  Compute entry points allocate nothing: scratch space comes from
 * the caller's workspace, sized by the *_workspace_size calls.  Work is
 * enqueued on `stream` (a hipStream_t; NULL is the null stream) and the call
 * returns without synchronising; nothing is copied between host and device.
 * The current HIP device is used.  Calls keep no global state: the only
 * state a call touches is what the caller passes in (buffers, and for the
 * layer call an optional kairos_context the caller created), so calls are
 * reentrant; calls that share output buffers on one stream are ordered by it.
 *
 * Errors: all arguments are validated on the host before anything is
 * enqueued.  An invalid call returns a negative kairos_status and has no side
 * effects.  A failed launch returns KAIROS_ERR_HIP; faults inside kernels
 * surface at the caller's next synchronisation.
 */
#ifndef KAIROS_H
#define KAIROS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KAIROS_OK = 0,
  KAIROS_ERR_NULL = -1,        /* a required pointer is NULL                      */
  KAIROS_ERR_SHAPE = -2,       /* a size is out of range or inconsistent          */
  KAIROS_ERR_DTYPE = -3,       /* unsupported element type                        */
  KAIROS_ERR_ALIGN = -4,       /* a buffer is not 16-byte aligned                 */
  KAIROS_ERR_ALIAS = -5,       /* an output overlaps an input it may not overlap  */
  KAIROS_ERR_UNSUPPORTED = -6, /* valid in principle, not implemented             */
  KAIROS_ERR_WORKSPACE = -7,   /* workspace missing or too small                  */
  KAIROS_ERR_HIP = -8,        /* a HIP launch or query failed                    */
  KAIROS_ERR_RANGE = -9       /* input values outside their range (reported by the
                                 binding's debug check, kairos_gdn_check_gates)   */
} kairos_status;

typedef enum {
  KAIROS_F32 = 0,
  KAIROS_BF16 = 1,
  KAIROS_FP8_E4M3 = 2,
  KAIROS_FP4_E2M1 = 3          /* 4-bit windowed Q/K: OCP FP4 E2M1 codes, two per byte */
} kairos_dtype;

/* Quantisation blocks of FP8 / 4-bit windowed Q and K (64 tokens each).
 *   KAIROS_QK_BLOCKS_TOKENS  consecutive 64-token blocks of the call (a block
 *                            may straddle two frames when 64 does not divide L)
 *   KAIROS_QK_BLOCKS_FRAMES  64-token blocks restarting at every frame (a
 *                            frame's last block holds L mod 64 tokens when 64
 *                            does not divide L); required for a streamed
 *                            rollout with quantised Q/K, which then quantises
 *                            exactly as one run over the whole sequence */
typedef enum { KAIROS_QK_BLOCKS_TOKENS = 0, KAIROS_QK_BLOCKS_FRAMES = 1 } kairos_qk_blocks;

/* Window form of the SWA / DSWA branches (Sec. 2.2.2, Eq. 7).
 *   KAIROS_WINDOW_CAUSAL    query i sees keys i - w < j <= i (w keys with itself)
 *   KAIROS_WINDOW_CENTERED  Eq. 7's centred band as printed: |j - i| <= floor(w / 2)
 *                           (keys on both sides, itself included; no streaming) */
typedef enum { KAIROS_WINDOW_CAUSAL = 0, KAIROS_WINDOW_CENTERED = 1 } kairos_window_kind;

/* Gated delta rule problem.  dk == dv == d with d in {32, 64, 128};
 * chunk must be 64 (the chunkwise evaluation's block length; any chunk size
 * gives the same result up to rounding).  io: KAIROS_F32 (q, k, v, out fp32,
 * token-by-token fp32 evaluation) or KAIROS_BF16 (q, k, v, out bf16, chunkwise
 * evaluation on bf16 matrix cores, fp32 state; d in {64, 128}).
 * B >= 1, H >= 1, T >= 0 (T == 0 copies state_in to state_out). */
typedef struct {
  int32_t B, T, H, dk, dv;
  int32_t chunk;
  int32_t io;                  /* kairos_dtype */
} kairos_gdn_desc;

/* Hybrid layer problem.  g describes q, k, v, alpha, beta, state (io must be
 * KAIROS_BF16, d == 128; H <= 65536, since the window kernel addresses a key
 * block's rows by 32-bit offsets).  The sequence is T tokens of frames of L tokens
 * (the last frame may be partial when ring_frames == 0).  window w >= 1 in
 * tokens; dilation >= 1.  frame_offset is the absolute index of the call's
 * first frame.  window_qk: KAIROS_BF16, or KAIROS_FP8_E4M3 / KAIROS_FP4_E2M1
 * to quantise the windowed branches' q and k per 64-token block, the blocks
 * laid out as qk_blocks says (kairos_qk_blocks; with a ring, quantised Q/K
 * need KAIROS_QK_BLOCKS_FRAMES, else KAIROS_ERR_UNSUPPORTED).
 * ring_frames R: 0 for a self-contained call (no keys before token 0);
 * otherwise the call continues a rollout: frames frame_offset-R ..
 * frame_offset-1 (those >= 0) are read from the ring, T must be a multiple of
 * L, and R must be >= kairos_hlta_ring_frames_required().  window_kind
 * (kairos_window_kind) applies to both windowed branches; a centred window
 * sees later frames, so it needs ring_frames == 0 (else
 * KAIROS_ERR_UNSUPPORTED); frame_offset still sets the DSWA residue groups.
 * rope_base: 0 for none, else RoPE (Sec. 2.2.2: every sliding-window block
 * uses rotary relative position encoding; RoFormer's definition: feature
 * pairs (2i, 2i+1) rotated by p * base^(-2i/d)) on the windowed branches' q
 * and k at each branch's positions p = (f div dil) * L + (t mod L), f the
 * absolute frame (SWA: the absolute token index; DSWA: the position in the
 * residue group's sub-sequence); applied before the FP8 quantisation; not on
 * the gated delta rule.  Positions are absolute, so a key rotated in one call
 * is the same key in every later call: with a ring, the ring keeps the
 * rotated keys (see kairos_hlta_fwd).
 * qk_blocks: kairos_qk_blocks (0, the former reserved field, keeps the
 * call's token order). */
typedef struct {
  kairos_gdn_desc g;
  int32_t L;
  int32_t window;
  int32_t dilation;
  int32_t window_qk;           /* kairos_dtype */
  int64_t frame_offset;
  int32_t ring_frames;
  int32_t window_kind;         /* kairos_window_kind */
  float rope_base;             /* 0: no RoPE; else > 0, finite (10000 is RoFormer's) */
  int32_t qk_blocks;           /* kairos_qk_blocks */
} kairos_hlta_desc;

/* Human-readable name of a status code (static storage). */
const char* kairos_status_string(int status);

/* ABI version: 100 * major + minor. */
int kairos_version(void);

/* Workspace bytes needed by kairos_gdn_fwd / kairos_hlta_fwd for this problem
 * (written to *bytes; 0 is a valid answer).  Validates the descriptor only. */
int kairos_gdn_workspace_size(const kairos_gdn_desc* desc, size_t* bytes);
int kairos_hlta_workspace_size(const kairos_hlta_desc* desc, size_t* bytes);

/* Ring frames a streamed (causal) call needs: dilation * ceil((window - 1) / L)
 * (frames whose keys a query can still see), written to *frames. */
int kairos_hlta_ring_frames_required(const kairos_hlta_desc* desc, int32_t* frames);

/* Bytes of the key ring and of the value ring of kairos_hlta_fwd for this
 * descriptor (ring_frames R > 0).  Layout: the value ring is [B][R][L][H][d]
 * bf16.  The key ring is P parts of k_part bytes each, P = 2 with RoPE and
 * dilation > 1 (part 0 keys rotated at SWA positions, part 1 at DSWA
 * positions), else 1; a part holds the key rows [B][R][L][H][row] (bf16, or
 * E4M3 / E2M1 codes of row d or d/2 bytes) and, for quantised keys, their
 * block scales [B][H][R][ceil(L/64)] fp32 at the next 256-byte boundary after
 * the rows (k_part then ends at a 256-byte boundary too).  For bf16 keys
 * without RoPE this is [B][R][L][H][d] bf16, as for the value ring. */
int kairos_hlta_ring_size(const kairos_hlta_desc* desc, size_t* k_bytes, size_t* v_bytes);

/* Gated delta rule forward (Sec. 2.2.1, Eq. 1-6 canonical form, step 4).
 *   q, k, v      [B][T][H][d]  io type; k L2-normalised per (token, head)
 *   alpha, beta  [B][T][H]     fp32, alpha in (0, 1], beta >= 0 (beta <= 1 for the
 *                canonical form; the printed Eq. 6 form of kairos_gdn_prologue
 *                passes beta / alpha, which may exceed 1)
 *   state_in     [B][H][d][d]  fp32 initial memory; NULL means zero
 *   out          [B][T][H][d]  io type, o_t = S_t q_t; must not overlap inputs
 *   state_out    [B][H][d][d]  fp32 final memory; NULL discards it; may equal
 *                state_in (in-place carry) but may not partially overlap it
 *   workspace    >= kairos_gdn_workspace_size bytes, 256-byte aligned (may be
 *                NULL when 0): the bf16 path keeps each chunk's T = (I + A)^{-1}
 *                and decays there (B*H*ceil(T/64)*(64*64*2 + 64*4) bytes) */
int kairos_gdn_fwd(const kairos_gdn_desc* desc, const void* q, const void* k, const void* v,
                   const float* alpha, const float* beta, const float* state_in,
                   void* out, float* state_out, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Debug check of the gates (Sec. 2.2.1: alpha and beta are sigmoids, Eq. 1
 * and Eq. 4; Sec. 2.3.2, Remark 2, Eq. 18: the long-horizon bound needs a
 * contractive update, which holds for alpha <= 1 and, with unit keys,
 * 0 <= beta <= 1; the kernels take log2 alpha, so alpha must be > 0).
 * Counts the (b, t, h) with alpha outside (0, 1] or beta outside
 * [0, beta_max] (NaN counts as outside) into *count.
 *   alpha, beta  [B][T][H] fp32, 16-byte aligned (may be NULL when T == 0)
 *   beta_max     1 for the canonical form; larger for the printed Eq. 6 form
 *                of kairos_gdn_prologue, whose beta / alpha may exceed 1
 *   count        one device uint32, 4-byte aligned, overwritten (not added to)
 * Enqueued on `stream` like every other call: the count is valid once the
 * stream reaches that point (the caller reads it).  Nothing else is touched.
 * Errors: KAIROS_ERR_NULL, _SHAPE (B, H < 1, T < 0, B*T*H above 2^40, NaN or
 * negative beta_max), _ALIGN, _ALIAS (count inside alpha or beta), _HIP. */
int kairos_gdn_check_gates(const float* alpha, const float* beta, int32_t B, int32_t T, int32_t H,
                           float beta_max, uint32_t* count, void* stream);

/* kairos_gdn_fwd for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation and kernels, with the workspace taken from a scratch array
 * the library holds in each device's memory (64 MiB, a fixed part of the
 * library's device image, kept until the process ends).  Calls nothing that
 * allocates.  Arguments and errors as for kairos_gdn_fwd, with no workspace
 * arguments; a problem whose workspace (kairos_gdn_workspace_size) exceeds
 * 64 MiB returns KAIROS_ERR_WORKSPACE.  The first call on a device resolves
 * that device's copy of the array (KAIROS_ERR_HIP if the runtime refuses).
 * All no-alloc calls on one device share its array: calls that overlap in
 * time on one device (concurrent streams or host threads) race and give
 * undefined results; calls ordered on one stream are safe. */
int kairos_gdn_fwd_noalloc(const kairos_gdn_desc* desc, const void* q, const void* k,
                           const void* v, const float* alpha, const float* beta,
                           const float* state_in, void* out, float* state_out, void* stream);

/* One windowed softmax branch on its own (Sec. 2.2.2): SWA when dilation == 1,
 * DSWA otherwise (Eq. 8 as a frame-residue index map; nothing is rearranged
 * in memory).  Uses desc->L, window, frame_offset, ring_frames, window_qk and
 * g.{B,T,H,dk}; `dilation` overrides desc->dilation.  With window_qk ==
 * KAIROS_FP8_E4M3 (KAIROS_FP4_E2M1), q and k are the codes and q_scales /
 * k_scales the per-64-token-block scales written by kairos_fp8_quantize
 * (kairos_fp4_quantize); otherwise q, k are bf16 and the scale pointers must
 * be NULL.  out [B][T][H][d] bf16.  The ring
 * is read, never written.  q and k are used as given: desc->rope_base must be
 * 0 (apply kairos_rope with the branch's dilation first). */
int kairos_window_fwd(const kairos_hlta_desc* desc, int32_t dilation, const void* q, const void* k,
                      const void* v, const float* q_scales, const float* k_scales,
                      const void* k_ring, const void* v_ring, void* out, void* stream);

/* Execution context of kairos_hlta_fwd, owned by the caller: a side stream
 * of the device current at creation (default priority, non-blocking) and
 * three events, with which a layer call runs part of its work beside the
 * caller's stream (see kairos_hlta_fwd).  kairos_context_create allocates
 * these host-side HIP objects (no device memory) and writes the handle to
 * *ctx (NULL on failure: KAIROS_ERR_NULL for ctx == NULL, KAIROS_ERR_HIP when
 * the runtime refuses).  kairos_context_destroy releases them (NULL is a
 * no-op); work already enqueued on the side stream still completes.  A
 * context may be shared by calls on several streams and host threads (an
 * internal lock orders its event pairs); destroy it only when no call that
 * uses it is running. */
typedef struct kairos_context_t* kairos_context;
int kairos_context_create(kairos_context* ctx);
int kairos_context_destroy(kairos_context ctx);

/* Hybrid layer forward: y = sig(z_swa) o_swa + sig(z_dswa) o_dswa + sig(z_gdn) o_gdn
 * per head (Sec. 2.2, Fig. 5 pathways, run as parallel gated branches).
 *   gate_logits  [3][H] fp32 (device memory)
 *   k_ring, v_ring  required iff ring_frames > 0, laid out and sized as
 *                kairos_hlta_ring_size says ([B][R][L][H][d] bf16 each for
 *                bf16 Q/K without RoPE); read for the frames before the call,
 *                then updated in stream order with the call's last min(R, F)
 *                frames.  The key ring holds the keys the windowed branches
 *                read: with RoPE the rotated keys, with quantised Q/K their
 *                codes and block scales; a rollout keeps L, window, dilation,
 *                rope_base, window_qk and qk_blocks fixed across its calls
 *   out          [B][T][H][d] bf16; state_out as in kairos_gdn_fwd
 *   workspace    >= kairos_hlta_workspace_size bytes
 *   ctx          NULL, or a context of the current device (else
 *                KAIROS_ERR_UNSUPPORTED)
 * Streams: with ctx == NULL everything runs on `stream`.  With a context,
 * part of the work runs on its side stream: the windowed branches' operand
 * pre-passes (quantised Q/K, RoPE) beside the GDN scan, or, when the window
 * kernel and the GDN scan fit on the device together (e.g. one streamed
 * frame), the whole GDN branch beside the window kernel.  The side stream
 * waits for an event recorded on `stream`, and `stream` waits for it before
 * anything that reads its results, so the call behaves as one stream and can
 * be captured into a graph.  While the side stream belongs to an open graph
 * capture, a call on a stream outside that capture runs on `stream` alone
 * (same results), so captures and eager calls on other threads can share a
 * context. */
int kairos_hlta_fwd(const kairos_hlta_desc* desc, const void* q, const void* k, const void* v,
                    const float* alpha, const float* beta, const float* gate_logits,
                    const float* state_in, void* k_ring, void* v_ring, void* out,
                    float* state_out, void* workspace, size_t workspace_bytes,
                    kairos_context ctx, void* stream);

/* The windowed stage of kairos_hlta_fwd on its own: both windowed branches
 * and the gated combination with an already computed GDN branch output.
 *   q, k       bf16 [B][T][H][128], or codes with q_scales / k_scales
 *              (window_qk == KAIROS_FP8_E4M3 / KAIROS_FP4_E2M1, as written by
 *              kairos_fp8_quantize / kairos_fp4_quantize)
 *   v          bf16 [B][T][H][128];  o_gdn bf16 [B][T][H][128]
 *   gate_logits [3][H] fp32;  k_ring / v_ring as in kairos_hlta_fwd (read only)
 *   out        bf16 [B][T][H][128], y = sig(z_swa) o_swa + sig(z_dswa) o_dswa + sig(z_gdn) o_gdn
 *   workspace  >= 4*B*T*H*129 bytes, 256-byte aligned (fp32 partial results:
 *              a row of 128 per query, then one log-sum-exp per query)
 * kairos_hlta_fwd = [kairos_fp8_quantize x2] + kairos_gdn_fwd + this call
 * [+ the ring update]; the stages are exposed for timing and composition.
 * Both branches share q and k, so desc->rope_base must be 0 here (with RoPE
 * the branches need differently rotated q, k: use kairos_hlta_fwd). */
int kairos_hlta_window_fwd(const kairos_hlta_desc* desc, const void* q, const void* k,
                           const void* v, const float* q_scales, const float* k_scales,
                           const void* o_gdn, const float* gate_logits, const void* k_ring,
                           const void* v_ring, void* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Flags of kairos_gdn_prologue. */
typedef enum {
  KAIROS_PROLOGUE_NORMALIZE_Q = 1,   /* also L2-normalise q                          */
  KAIROS_PROLOGUE_LITERAL_EQ6 = 2    /* emit the inputs of the printed Eq. 6 form    */
} kairos_prologue_flags;

/* Input prologue of the gated delta rule: turns raw per-token keys and gate
 * logits into the inputs kairos_gdn_fwd / kairos_hlta_fwd take (Sec. 2.2.1:
 * Eq. 1 beta = sig(z_beta); Eq. 4 alpha = sig(z_alpha); Eq. 2-3 take unit
 * keys).  Per (token, head) row:
 *   k_out     = k_in / ||k_in||_2                  (a zero row stays zero)
 *   q_out     = q_in / ||q_in||_2                  with KAIROS_PROLOGUE_NORMALIZE_Q
 *   alpha_out = sig(alpha_logits)
 *   beta_out  = sig(beta_logits)
 * With KAIROS_PROLOGUE_LITERAL_EQ6 the outputs make the canonical recurrence
 * equal to Eq. 6 as printed (erasing with the un-decayed retrieval
 * S_{t-1} k_t): beta_out = sig(beta_logits) / sig(alpha_logits) and
 * v_out = sig(alpha_logits) * v_in (rounded to the io type); alpha_out is
 * unchanged.  That form needs sig(alpha_logits) > 0 in fp32: alpha_logits
 * >= -80; below, beta_out overflows.
 *   desc          as for kairos_gdn_fwd (io KAIROS_F32 or KAIROS_BF16); only
 *                 B, T, H, dk and io are used; chunk must still be 64
 *   k_in, k_out   [B][T][H][d] io type
 *   alpha_logits, beta_logits, alpha_out, beta_out   [B][T][H] fp32
 *   q_in, q_out   [B][T][H][d] io type with KAIROS_PROLOGUE_NORMALIZE_Q, else NULL
 *   v_in, v_out   [B][T][H][d] io type with KAIROS_PROLOGUE_LITERAL_EQ6, else NULL
 * Arithmetic is fp32 (the norm after an exact power-of-two rescaling of each
 * row by its largest magnitude, so tiny or huge rows still normalise);
 * bf16 outputs are rounded to nearest even.  Inputs must be finite.  Each
 * output may be the same buffer as its own input (in place: k_out == k_in,
 * alpha_out == alpha_logits, ...); any other overlap is KAIROS_ERR_ALIAS.
 * A pointer given for a tensor its flag does not ask for is
 * KAIROS_ERR_UNSUPPORTED, as is an unknown flag bit.  T == 0 does nothing. */
int kairos_gdn_prologue(const kairos_gdn_desc* desc, int32_t flags, const void* k_in,
                        const float* alpha_logits, const float* beta_logits, const void* q_in,
                        const void* v_in, void* k_out, float* alpha_out, float* beta_out,
                        void* q_out, void* v_out, void* stream);

/* RoPE of one windowed branch's q or k (Sec. 2.2.2; definition as for
 * kairos_hlta_desc.rope_base) at the positions of the branch with the given
 * dilation (1: SWA, the absolute token index; > 1: DSWA, the position in the
 * residue group's sub-sequence), using desc->{g.B, g.T, g.H, g.dk, L,
 * frame_offset, rope_base (> 0), window_qk}.
 *   x       [B][T][H][d] bf16
 *   out     window_qk == KAIROS_BF16: [B][T][H][d] bf16, may be x itself (in
 *           place); KAIROS_FP4_E2M1: E2M1 codes [B][T][H][d/2] bytes of the
 *           rotated values, quantised as kairos_fp4_quantize does;
 *           KAIROS_FP8_E4M3: E4M3 codes [B][T][H][d] uint8 of the
 *           rotated values, quantised as kairos_fp8_quantize does
 *   scales  FP8 / FP4: [B][H][ceil(T/64)] fp32; bf16: must be NULL
 * Angles are reduced in fp64, cos/sin in fp32, the rotation in fp32; bf16
 * output rounds to nearest even.  kairos_rope + kairos_window_fwd per branch
 * equals the windowed branches of kairos_hlta_fwd with RoPE. */
int kairos_rope(const kairos_hlta_desc* desc, int32_t dilation, const void* x, void* out,
                float* scales, void* stream);

/* 4-bit quantisation of x [B][T][H][d] bf16 per (b, h, 64-token block), the
 * INT4 attention quantisation of the project page (Sec. 2, Q2) as OCP FP4
 * E2M1 codes (the matrix instructions take 4-bit floating-point operands, not
 * 4-bit integers): s = amax / 6 (fp32; 1 when amax == 0), code = E2M1 of the
 * correctly rounded fp32 quotient x / s, round to nearest with ties to the
 * even code, saturating at 6.  codes [B][T][H][d/2] bytes, feature 2i in the
 * low nibble of byte i; scales [B][H][ceil(T/64)] fp32.  d in {32, 64, 128}.
 * Errors as for kairos_fp8_quantize. */
int kairos_fp4_quantize(const void* x_bf16, uint8_t* codes, float* scales, int32_t B, int32_t T,
                        int32_t H, int32_t d, void* stream);

/* FP8 E4M3 quantisation of x [B][T][H][d] bf16 per (b, h, 64-token block),
 * the FP8 attention quantisation of the project page (Sec. 2, Q2: FP8/INT4
 * attention quantisation in the deployment co-design; Sec. 1 TL;DR: FP8
 * inference):
 * s = amax / 448 (fp32; 1 when amax == 0), code = E4M3(x / s) with an IEEE
 * fp32 division, round to nearest even, saturating at 448 (OCP E4M3: bias 7,
 * subnormals, no infinities).  codes [B][T][H][d] uint8, scales
 * [B][H][ceil(T/64)] fp32.  d in {32, 64, 128}. */
int kairos_fp8_quantize(const void* x_bf16, uint8_t* codes, float* scales, int32_t B, int32_t T,
                        int32_t H, int32_t d, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KAIROS_H */
