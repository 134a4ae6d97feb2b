/*
 * jagged_attn.h -- C ABI of the MI355X (gfx950) jagged generalized dot-product
 * attention library (libjagged_attn.so): the forward, its backward for
 * training, and an on-device MX (e4m3 + E8M0) quantiser.
 *
 * What it computes.  For every sample b and head h of a jagged batch, with
 * Q (Lq x D) and K, V (Lk x D) the sample's rows of that head:
 *   softmax:    O = softmax(Q K^T / sqrt(D)) V over the allowed keys;
 *   gelu_tanh:  O = gelu_tanh(rms(Q) rms(K)^T / sqrt(D)) V / Lk, where rms()
 *               is unit-weight RMSNorm per token and head (the QK-norm that
 *               bounds the activation input) and there is no max and no sum.
 * Sources: techfeed.io summary of "GEM Training: How Meta Doubled the
 * Efficiency of Its LLM-Scale Ads Foundation Model", sections "なぜLLM向けの
 * インフラをそのまま使えないのか" (jagged histories; the three shapes: self with a
 * short window, cross with long Q / short K,V, PMA with short Q / long K,V),
 * "Generalized Dot-Product Attention（GDPA）" (one kernel for the three shapes,
 * GELU with QK-norm), "BlockAttention" (fixed 64-token blocks, window a whole
 * number of blocks) and "MXFP8による超低精度トレーニング" (microscaling FP8
 * attention); remio.ai "Meta Engineering、広告モデルの拡大とともにGEMの学習効率を
 * 2倍にしたと説明", section "効率向上はモデルとシステムの協調設計から生まれた" (GDPA
 * replaces softmax by other activations).
 *
 * Readings where the pages are silent: no causal mask (window 0 = full
 * attention over the sample's keys); scale 1/sqrt(D) everywhere; a window W>0
 * lets a query in 64-token block i see every key of blocks i-W/64+1 .. i, with
 * blocks counted from the sample's first token; Lk == 0 gives O == 0.
 * JA_SLIDING is the token-level sliding window that block attention grew out
 * of ("BlockAttention" section: O(L x window) self-attention): query i sees
 * keys i-W+1 .. i, positions counted from the sample's first token.
 *
 * Layouts (all device memory, row-major, contiguous):
 *   q   [total_q , H, D]     k, v [total_kv, H, D]     out [total_q, H, D]
 *   element type by io->dtype: JA_F32 -> float in and out;
 *   JA_BF16 -> bfloat16 in and out; JA_MXFP8_E4M3 -> e4m3 ("fn") bytes in,
 *   with E8M0 scale bytes q_scale/k_scale/v_scale [rows, H, D/32] (one scale
 *   per 32 contiguous elements along D), bfloat16 out.
 *   q_offsets, kv_offsets: device int32 [B+1], offsets[0] == 0, non-decreasing,
 *   offsets[B] == total_q / total_kv.  Sample b owns rows [off[b], off[b+1]).
 *   JA_SELF and JA_SLIDING need q_offsets and kv_offsets to hold the same
 *   values (the same pointer may be passed twice).  Buffers need 16-byte
 *   alignment.  In jagged_attn_fwd, q, out and q_scale may be NULL when
 *   total_q == 0, and k, v, k_scale and v_scale when total_kv == 0 (empty
 *   tensors); in jagged_attn_bwd likewise q, dout and dq, and k, v, dk and
 *   dv; the offsets are always required.
 *
 * Ownership.  The caller owns every buffer, including the workspace.  The
 * library allocates nothing inside jagged_attn_fwd and keeps only a per-device
 * cache of device properties.  Calls on different streams with different
 * workspaces and outputs are independent; calls sharing a workspace must be
 * ordered on one stream.
 *
 * Errors.  Every entry point returns JA_OK (0) or a negative ja_status.
 * Argument errors are detected on the host before anything is launched.
 * jagged_attn_fwd is asynchronous on io->stream and never synchronises; the
 * offsets are validated on the device, which writes a status word into the
 * workspace and then skips all work (out is left unspecified); read it with
 * jagged_attn_check.  Output contents are unspecified whenever the status is
 * not JA_OK.
 *
 * Debug mode.  With the environment variable JA_DEBUG set to anything but
 * "0" (read once per process), jagged_attn_fwd, jagged_attn_fwd_noalloc,
 * jagged_attn_bwd and jagged_attn_mx_quantize synchronise their stream before
 * returning and return the device status themselves: JA_EOFFSETS for offsets
 * the device rejected, JA_EHIP for a launch or runtime fault, else JA_OK.
 */
#ifndef JAGGED_ATTN_H
#define JAGGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum ja_variant {
  JA_SELF = 0,  /* q and kv share offsets; optional block window            */
  JA_CROSS = 1, /* long queries, short keys/values: work split by q tiles    */
  JA_PMA = 2,   /* short queries (<=32 per sample), long keys/values: work
                   split by key chunks, partial results merged on device      */
  JA_SLIDING = 3 /* self-attention with a token sliding window: window = W >= 1
                   keys ending at the query; JA_SOFTMAX, JA_F32 or JA_BF16     */
};

enum ja_act {
  JA_SOFTMAX = 0,   /* softmax over the allowed keys                         */
  JA_GELU_TANH = 1, /* QK-RMSNorm, gelu_tanh score, 1/Lk normalisation        */
  JA_GELU_POLY = 2  /* as JA_GELU_TANH with tanh replaced by an ALU-only
                       polynomial (GDPA section: the ALU GELU; here a fitted
                       even polynomial on |x| < 4, x or 0 outside; max error
                       of the activation about 2e-4)                          */
};

enum ja_dtype { JA_F32 = 0, JA_BF16 = 1, JA_MXFP8_E4M3 = 2 };

enum ja_status {
  JA_OK = 0,
  JA_EINVAL = -1,       /* bad argument (null pointer, B<1, H<1, bad enum...)  */
  JA_EUNSUPPORTED = -2, /* valid but not implemented (D not in {32,64,128},
                           windowed GELU, window not a multiple of 64,
                           JA_SLIDING with MXFP8 ...)                          */
  JA_EWORKSPACE = -3,   /* workspace missing or smaller than required         */
  JA_EHIP = -4,         /* a HIP runtime call or kernel launch failed         */
  JA_EOFFSETS = -5      /* device found offsets that are not monotone, do not
                           start at 0, do not end at total, or (JA_SELF,
                           JA_SLIDING) differ                                  */
};

typedef struct ja_io {
  int dtype;                 /* enum ja_dtype                                  */
  const uint8_t *q_scale;    /* JA_MXFP8_E4M3 only: E8M0 [total_q , H, D/32]    */
  const uint8_t *k_scale;    /*                     E8M0 [total_kv, H, D/32]    */
  const uint8_t *v_scale;    /*                     E8M0 [total_kv, H, D/32]    */
  void *workspace;           /* device memory, >= jagged_attn_workspace_size() */
  size_t workspace_bytes;
  void *stream;              /* hipStream_t to launch on; NULL = null stream    */
  int32_t total_q;           /* rows of q/out  (= q_offsets[B])                 */
  int32_t total_kv;          /* rows of k/v    (= kv_offsets[B])                */
  float rms_eps;             /* GELU acts: RMSNorm epsilon; <= 0 -> 1e-6        */
  void *ev_start;            /* optional profiling hipEvent_t pair (or NULL):   */
  void *ev_stop;             /* written by the attention kernel's own dispatch  */
                             /* (its start and end; not the plan or the         */
                             /* split-merge kernel), so the kernel can be timed */
                             /* without a profiler and without extra packets    */
  int32_t max_workgroups;    /* 0: the library's choice (every resident slot of */
                             /* the device); > 0: at most this many workgroups  */
                             /* for the attention kernel, rounded down to a     */
                             /* multiple of 8 (at least 8), e.g. to leave CUs   */
                             /* to concurrent work.  Results are bitwise        */
                             /* identical for every grid.  < 0: JA_EINVAL       */
  int32_t *status;           /* optional device int32 owned by the caller (4-B  */
                             /* aligned): the device writes the call's status   */
                             /* word (JA_OK or JA_EOFFSETS) there as well, on   */
                             /* the stream, so it can be read back without      */
                             /* jagged_attn_check; NULL: not written            */
  uint64_t *softmax_stats;   /* optional device uint64[3], diagnostics: when    */
                             /* non-NULL the tile-stream softmax (bf16 and MX   */
                             /* self- and cross-attention) adds, per wave and   */
                             /* 64-key tile, 1 to [0] (tiles), and 1 to [1] when */
                             /* it had to find the tile's max because the rows  */
                             /* had no reference yet (a query block's first     */
                             /* tile) or to [2] when a later tile moved the     */
                             /* reference up and rescaled O; other kernels and  */
                             /* the caller's zeroing: untouched.  Each wave adds */
                             /* its counts once, when it ends.                  */
  int32_t fp8_pv;            /* JA_MXFP8_E4M3 only: nonzero runs O += P V on    */
                             /* the block-scaled fp8 MFMA too ("MXFP8..."       */
                             /* section: attention in microscaling fp8).  V is  */
                             /* requantised per tile along the keys (scale of a */
                             /* 32-key x 32-dim block = the largest of its keys' */
                             /* MX scales, codes shifted down and rounded to    */
                             /* nearest even) and P per query and 32 keys       */
                             /* (scale 2^(floor(log2 max) - 7)); the row sum    */
                             /* adds the quantised weights.  Less exact than    */
                             /* the default (V exact in bf16, P in bf16).       */
                             /* Not available in this version: every call with */
                             /* it set returns JA_EUNSUPPORTED.                 */
  float *lse;                /* optional device float32 [total_q, H] owned by   */
                             /* the caller (4-byte aligned), softmax only: the  */
                             /* forward writes, per query row and head, the     */
                             /* natural log-sum-exp of its scaled scores over   */
                             /* the keys the row attends,                       */
                             /* log sum_j exp(q.k_j / sqrt(D)), or -inf for a   */
                             /* row without keys.  Every fp32 and bf16 call,    */
                             /* and MXFP8 PMA and self-attention at D = 128     */
                             /* (full, or windows of up to four blocks); the    */
                             /* other MXFP8 calls with it set return            */
                             /* JA_EUNSUPPORTED, GELU calls JA_EINVAL.  NULL:   */
                             /* not written.                                    */
                             /* jagged_attn_bwd reads it instead (see there).   */
  const void *fwd_out;       /* jagged_attn_bwd only, optional: the forward's   */
                             /* output for the same arguments ([total_q, H, D], */
                             /* the input dtype, 16-byte aligned), given with   */
                             /* lse; jagged_attn_fwd ignores it.                */
} ja_io;

/* The forward pass.  Arguments as described above; window is 0 (no window) or
 * a positive multiple of 64 (JA_SELF + JA_SOFTMAX only), or for JA_SLIDING
 * the window in tokens (>= 1, required). */
int jagged_attn_fwd(const void *q, const void *k, const void *v,
                    const int32_t *q_offsets, const int32_t *kv_offsets,
                    int B, int H, int D, int variant, int act, int window,
                    void *out, const ja_io *io);

/* jagged_attn_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops and harnesses that forbid allocation): the
 * same computation, arguments and errors, except that io->workspace must be
 * NULL and io->workspace_bytes 0 (JA_EINVAL otherwise).  The workspace is the
 * library's own device array of 64 MiB, one per GPU the library runs on, held
 * until the process ends; a call whose jagged_attn_workspace_size() exceeds
 * 64 MiB returns JA_EWORKSPACE before anything is launched.  The first call
 * on a device looks the array's address up on that device (device ids 0..63;
 * others give JA_EUNSUPPORTED).  Nothing is allocated, on the host or the
 * device.  Every call on one GPU shares that GPU's array, which keeps the
 * last call's contents (no call needs it cleared): calls that overlap on one
 * GPU -- on different streams, or from different threads -- race and must be
 * ordered by the caller.  Device-detected offset errors are reported through
 * io->status (jagged_attn_check needs a caller workspace). */
int jagged_attn_fwd_noalloc(const void *q, const void *k, const void *v,
                            const int32_t *q_offsets, const int32_t *kv_offsets,
                            int B, int H, int D, int variant, int act, int window,
                            void *out, const ja_io *io);

/* Bytes of workspace jagged_attn_fwd needs for these arguments (0 on invalid
 * arguments).  Depends on the arguments only, not on the device. */
size_t jagged_attn_workspace_size(int B, int H, int D, int variant, int act,
                                  int window, int dtype, int32_t total_q,
                                  int32_t total_kv);

/* Backward of the forward, for training (the pages describe the training
 * system but not its backward; this is the chain-rule derivative of the
 * forward as defined above).  For every sample and head:
 *   JA_SOFTMAX, with P the softmax weights of the forward:
 *     dV = P^T dO,  dS = P * (dO V^T - rowsum(P * (dO V^T))),
 *     dQ = dS K / sqrt(D),  dK = dS^T Q / sqrt(D);
 *   JA_GELU_TANH, with Qn, Kn the RMS-normalised rows, S = Qn Kn^T / sqrt(D):
 *     dV = gelu(S)^T dO / Lk,  dS = gelu'(S) * (dO V^T) / Lk,
 *     dQn = dS Kn / sqrt(D),  dKn = dS^T Qn / sqrt(D), then through the
 *     RMSNorm row by row: dx = r dxn - x r^3 (dxn . x) / D,
 *     r = (mean(x^2) + eps)^(-1/2), eps = io->rms_eps (<= 0 -> 1e-6).
 * q, k, v: as for jagged_attn_fwd; dout: the gradient of out, laid out and
 * typed like q (JA_F32 or JA_BF16).  Writes float32 dq [total_q, H, D] and
 * dk, dv [total_kv, H, D] (every row written; rows of samples without keys
 * get zeros in dq, keys no query sees get zeros).  act: JA_SOFTMAX or
 * JA_GELU_TANH; variant, window and offsets as for jagged_attn_fwd (JA_SELF
 * with or without a block window, JA_SLIDING, JA_CROSS, JA_PMA; no window
 * with GELU).  Nothing from the forward is needed: row statistics and RMS
 * factors are recomputed.  A softmax call may hand over the forward's
 * io->lse and io->fwd_out (both or neither; JA_EINVAL otherwise, and for GELU
 * acts): the backward then takes each row's log-sum-exp from lse and
 * D_i = sum_j P_ij dP_ij as dO_i . O_i from fwd_out, and skips the pass over
 * the keys that recomputes them.  The gradients are those of the softmax
 * with that log-sum-exp; O rounded to bf16 moves D_i by about 2^-9 of
 * |dO_i| |O_i|.  Workspace of jagged_attn_bwd_workspace_size()
 * bytes in io->workspace; io->ev_start / ev_stop, when set, bracket the
 * gradient kernels (recorded around them on the stream); io->status as for
 * jagged_attn_fwd; io->max_workgroups is not used.  Asynchronous on io->stream; errors as for
 * jagged_attn_fwd (JA_EUNSUPPORTED for JA_GELU_POLY and MXFP8; offset errors
 * through jagged_attn_check). */
int jagged_attn_bwd(const void *q, const void *k, const void *v, const void *dout,
                    const int32_t *q_offsets, const int32_t *kv_offsets,
                    int B, int H, int D, int variant, int act, int window,
                    float *dq, float *dk, float *dv, const ja_io *io);

/* Bytes of workspace jagged_attn_bwd needs (0 on invalid arguments). */
size_t jagged_attn_bwd_workspace_size(int B, int H, int D, int variant, int act,
                                      int window, int dtype, int32_t total_q,
                                      int32_t total_kv);

/* MX quantisation on the device ("MXFP8による超低精度トレーニング" section:
 * attention on microscaling FP8 inputs; the page gives no encoding rule, the
 * one used is stated here).  x holds `rows` rows of D values, row-major and
 * contiguous (for attention inputs rows = tokens x heads), as float32
 * (dtype JA_F32) or bfloat16 (JA_BF16).  Writes codes [rows, D] (e4m3 "fn"
 * bytes) and scales [rows, D/32] (E8M0 bytes): per 32 contiguous elements of a
 * row, E = floor(log2(max |x|)) - 8 clamped to [-127, 127] (-127 for an
 * all-zero block), scale byte E + 127, and each code the e4m3 value nearest
 * to x / 2^E (ties to even) after saturating to +-448; NaN inputs are not
 * supported.  The output is the exact input of jagged_attn_fwd with
 * JA_MXFP8_E4M3.  All pointers are device memory owned by the caller, 16-byte
 * aligned (and may be NULL when rows == 0: nothing is done); nothing is
 * allocated.  Asynchronous on `stream` (a hipStream_t or
 * NULL).  Returns JA_OK, JA_EINVAL (null or misaligned pointer, rows < 0, D not
 * a positive multiple of 32, dtype not JA_F32/JA_BF16) or JA_EHIP. */
int jagged_attn_mx_quantize(const void *x, int dtype, int64_t rows, int D,
                            uint8_t *codes, uint8_t *scales, void *stream);

/* Synchronises `stream` (a hipStream_t or NULL) and returns the device status
 * word the last jagged_attn_fwd on this workspace wrote: JA_OK or
 * JA_EOFFSETS; JA_EHIP / JA_EINVAL if it cannot be read. */
int jagged_attn_check(const void *workspace, void *stream);

/* Static description of a status code; never NULL. */
const char *jagged_attn_strerror(int status);

/* Library ABI version (major*100 + minor). */
int jagged_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* JAGGED_ATTN_H */
