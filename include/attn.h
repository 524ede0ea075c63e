/*
 * attn.h -- C ABI of the fused exact-attention library for AMD MI355X (gfx950).
 *
 * The operation.  Exact scaled-dot-product attention, the computation that the
 * FlashAttention-4 pages are about ("英伟达最强B200算力浪费60%", QbitAI; and the
 * Tencent Cloud article "AI Infra 系列 第六章 GPU 性能工程（二）", section 7, FA4's
 * four techniques).  Per (batch b, head h) and query row i:
 *
 *     s_ij  = scale * sum_d Q[b,h,i,d] * K[b,h,j,d]      for visible keys j
 *     O_i   = sum_j softmax_j(s_ij) * V[b,h,j,:]
 *     LSE_i = ln sum_j exp(s_ij)                          (natural log)
 *
 * Visible keys: every j in [0, S), or only j <= i when `causal` is nonzero.  The
 * S x S score matrix never reaches memory: it is built tile by tile on chip with
 * an online softmax (the pages: section 7 of the Tencent Cloud article, and
 * section 5's tiling/fusion levers).  The backward computes dQ, dK, dV of the
 * same function, recomputing the probabilities from LSE instead of storing
 * them (section 5's recomputation lever).
 *
 * Conventions shared by every entry point.
 *   - Tensors are contiguous, row-major [B][H][S][D]: element (b,h,i,d) sits at
 *     ((b*H + h)*S + i)*D + d.  Q, K, V, O, dO, dQ, dK, dV are bf16 (16-bit
 *     brain float, passed as raw 16-bit words); LSE is fp32 [B][H][S].
 *   - All tensor pointers are DEVICE pointers on the current HIP device, owned
 *     by the caller.  The library allocates no device memory when called; the
 *     backward's scratch space is a caller-provided workspace (attn_bwd_noalloc
 *     instead uses a fixed array inside the library, described there).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without synchronising.  Errors raised while the kernels
 *     run surface at the caller's next synchronisation on that stream.
 *   - Arguments are validated on the host before any HIP call.  No C++
 *     exception crosses this boundary.  Calls are thread-safe and re-entrant
 *     (attn_bwd_noalloc calls that overlap on one GPU share its array: see
 *     there).
 *   - Supported: B, H, S >= 1 (any S; partial tiles are masked), D in {64, 128},
 *     B*H*S*D < 2^40 elements, S*D < 2^29, and B*H*ceil(S/256) < 2^23 (the
 *     kernels run one workgroup per 256-row block on a one-dimensional grid,
 *     whose work-item count must stay below 2^32).
 *   - Scale: any finite scale whose product with log2(e) is finite (|scale| <
 *     about 2.36e38; others return ATTN_ERR_SCALE).  The kernels form each
 *     score as an fp32 dot product multiplied by |scale| * log2(e), so the
 *     inputs must also keep |scale * q_i . k_j| * log2(e) below FLT_MAX
 *     (about 3.4e38) for every visible pair: a score past that overflows to
 *     infinity and the rows it touches come out NaN.  The one other
 *     data-dependent limit is |V| < 2^47 for the forward (see attn_fwd);
 *     unit-variance inputs sit many orders of magnitude inside both.
 *   - Every load stays inside the extent of the tensor it reads (a partial
 *     last tile is zero-filled on chip), so buffers may be allocated to their
 *     exact size with nothing mapped after them.
 *   - Arithmetic: bf16 inputs, fp32 accumulation in the matrix cores, fp32
 *     softmax statistics, outputs rounded to nearest-even.
 */
#ifndef EXACT_ATTN_H
#define EXACT_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t (HIP's stream handle), without needing HIP headers. */
typedef struct ihipStream_t* attn_stream_t;

/* Status codes returned by every entry point. */
enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL                         */
  ATTN_ERR_SHAPE = 2,       /* B, H or S < 1, B*H*S*D >= 2^40, S*D >= 2^29, or
                               B*H*ceil(S/256) >= 2^23                           */
  ATTN_ERR_HEAD_DIM = 3,    /* D is not 64 or 128                                 */
  ATTN_ERR_ALIGN = 4,       /* a bf16 tensor not 16-byte aligned, LSE not 4-byte,
                               or the workspace not 256-byte aligned              */
  ATTN_ERR_WORKSPACE = 5,   /* workspace smaller than attn_bwd_workspace_size()   */
  ATTN_ERR_SCALE = 6,       /* scale or scale*log2(e) not finite, or a rescale
                               threshold out of range                            */
  ATTN_ERR_UNSUPPORTED = 7, /* a valid request this build does not implement      */
  ATTN_ERR_HIP = 8,         /* the HIP runtime refused the launch; see
                               attn_last_hip_error()                              */
  ATTN_ERR_SCRATCH = 9      /* attn_bwd_noalloc: the shape needs more workspace
                               than attn_noalloc_scratch_bytes()                  */
};

/*
 * Forward: O and LSE of exact attention (definition above).
 *   q, k, v  [B][H][S][D] bf16, read only.
 *   o        [B][H][S][D] bf16, written.  May not alias q, k or v.
 *   lse      [B][H][S] fp32, written: the natural-log log-sum-exp of each
 *            row's scaled, visible logits (what the backward consumes).
 *   scale    multiplies the logits before masking and softmax (usually 1/sqrt(D)).
 *   causal   nonzero: key j is visible to query i iff j <= i.
 * The online softmax rescales the running output only when a row's maximum
 * grows by about 64 (log2 units) over the stale maximum it is using (the test
 * is described at attn_fwd_ex), the conditional-rescaling idea of FA4
 * (Tencent Cloud article, section 7): the unnormalised weights stay below
 * 2^64 and a row's sums below 2^81, inside the fp32 and bf16 exponent range
 * of the sums and the PV product as long as |V| < 2^47 (the fp32 output
 * accumulators hold at most 2^81 * max|V|).  The threshold and the
 * exponential policy come from a per-shape table (attn_fwd_default_policy);
 * the result is the same for every threshold, see attn_fwd_ex.
 * Returns ATTN_OK or an attn_status code; nothing is written on error.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int S, int D, float scale, int causal,
             attn_stream_t stream);

/*
 * Forward with an explicit rescale threshold `rescale_log2` in [0, 64]:
 * a wave of 32 query rows rescales its running outputs after a 128-key step
 * when some lane's sum of the step's weights, taken against the stale row
 * maximum, exceeds 2^rescale_log2.  That happens whenever a row maximum has
 * grown by more than rescale_log2 (in units of log2) past the maximum in
 * use, and may happen a little earlier (many weights close to the bound);
 * 0 rescales at every growth and on most steps besides.  Every threshold
 * yields the same exact result up to rounding (the stale maximum cancels
 * between numerator and denominator).  Other arguments as attn_fwd.
 * Out-of-range threshold: ATTN_ERR_SCALE.
 */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int S, int D, float scale, int causal,
                float rescale_log2, attn_stream_t stream);

/*
 * Forward with both softmax knobs explicit: the rescale threshold
 * rescale_log2 in [0, 64] (as attn_fwd_ex) and the exponential policy of FA4
 * (Tencent Cloud article, section 7: a polynomial exp2 on the FMA units for a
 * share of the elements, beside the hardware transcendental unit):
 *   exp_poly_every  0: every exponential on the hardware unit (v_exp_f32);
 *                   4 or 8: every 4th or 8th exponential of a lane (25 % or
 *                   12.5 % of them, a fixed column subset of each score
 *                   tile) by 2^floor(x) * p(x - floor(x)), p a cubic with
 *                   relative error below 8.6e-5 (23 times below the bf16
 *                   rounding the weights undergo next).
 * Every policy yields the same exact result up to rounding.  Sequences of at
 * most 128 keys take the one-pass short-sequence kernel, which has neither
 * knob (exact row maxima, hardware exponentials).  Other arguments as
 * attn_fwd.  Threshold out of range: ATTN_ERR_SCALE; exp_poly_every not 0, 4
 * or 8: ATTN_ERR_UNSUPPORTED.
 */
int attn_fwd_policy(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int S, int D, float scale, int causal,
                    float rescale_log2, int exp_poly_every, attn_stream_t stream);

/*
 * The policy attn_fwd picks for a shape (a table of measured winners per
 * shape; attn_fwd_ex keeps its exponential policy and takes the threshold
 * from the caller): writes the rescale threshold and the exponential policy
 * (as attn_fwd_policy).  NULL output: ATTN_ERR_NULL; D not 64 or 128:
 * ATTN_ERR_HEAD_DIM; S < 1: ATTN_ERR_SHAPE.
 */
int attn_fwd_default_policy(int D, int causal, int S, float* rescale_log2, int* exp_poly_every);

/*
 * FP8 forward: the same O and LSE for Q, K, V given as OCP FP8 E4M3 codes
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; 0x7f/0xff NaN,
 * largest finite 448) with one descale factor per tensor: the inputs are
 * Q = q_descale * value(q codes), and likewise K and V.  The precision lever
 * of the Tencent Cloud article, section 5, on the gfx950 FP8 matrix core:
 * both products run in E4M3 with fp32 accumulation.
 *   q, k, v    [B][H][S][D] E4M3 codes (one byte each), 16-byte aligned.
 *   o          [B][H][S][D] bf16, written (v_descale applied).
 *   lse        [B][H][S] fp32, written (natural log, as attn_fwd).
 *   q_descale, k_descale, v_descale   finite and > 0.
 * Arithmetic: the score products are exact (E4M3 x E4M3 fits fp32) and summed
 * in fp32; the softmax weights are rounded to E4M3 (to nearest even, relative
 * error <= 2^-4, weights under 2^-10 of a row's largest times 4 flushed to
 * zero) before the PV product, and O is normalised by the sum of exactly those
 * rounded weights, so each output row is a convex combination of V rows; the
 * LSE takes the fp32 sum of the unrounded weights.  Every row's O therefore
 * sits within (2^-4 / (1 - 2^-4)) * sum_j P_ij |V_j - O_i| (plus the flushed
 * weights' share and the bf16 output rounding) of the exact result on the
 * dequantized inputs; the LSE within the bf16 path's bound.  Sequences of
 * any length take the same kernel.  Errors as attn_fwd; a descale factor not
 * finite and positive, or scale * q_descale * k_descale * log2(e) not finite:
 * ATTN_ERR_SCALE.
 */
int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int S, int D, float scale, int causal, float q_descale,
                 float k_descale, float v_descale, attn_stream_t stream);

/*
 * Diagnostic forward that also counts the conditional-rescale events (the FA4
 * technique of rescaling only when the maximum threatens the number range,
 * Tencent Cloud article, section 7).  The kernel tests once per wave (32
 * query rows) and 128-key step after the row block's first step; a test fires
 * when some lane's sum of the step's weights, taken against the stale
 * maximum, exceeds 2^rescale_log2 — then the wave's maxima move up, O and the
 * sums are rescaled and the step's weights recomputed.
 *   events   device pointer to two unsigned 64-bit counters, 8-byte aligned,
 *            owned by the caller, who zeroes them: the launch ADDS the number
 *            of tests to events[0] and the number that fired to events[1].
 * Computes the same O and LSE as attn_fwd_ex with the same arguments, bit for
 * bit.  Other arguments and errors as attn_fwd_ex; events == NULL:
 * ATTN_ERR_NULL.
 */
int attn_fwd_rescale_events(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int S, int D, float scale, int causal,
                            float rescale_log2, unsigned long long* events,
                            attn_stream_t stream);

/*
 * Bytes of device workspace attn_bwd needs for this shape (0 if the shape is
 * invalid): a 16-byte record of two row statistics per query row,
 * -LSE_i * log2(e) and -Delta_i = -sum_d dO_id * O_id, each as three bf16
 * parts that sum to it in fp32 ([B][H][64 * ceil(S/64)][8] bf16, i.e. 1 KiB
 * per 64-row block), rounded up to 256 bytes.  A convention of this library, not of
 * the pages, which describe no interface: the caller owns every buffer, so
 * the backward's scratch space is passed in.  (The statistics themselves are
 * the backward's row sums Delta_i and the recomputation from LSE that the
 * definition above implies.)
 */
size_t attn_bwd_workspace_size(int B, int H, int S, int D);

/*
 * Backward: gradients of sum(dO * O) for the forward above.
 *   q, k, v      the forward's inputs (bf16 [B][H][S][D]).
 *   o, lse       the forward's outputs (bf16 O, fp32 LSE) for the same inputs.
 *   dout         dO, bf16 [B][H][S][D].
 *   dq, dk, dv   bf16 [B][H][S][D], written.  Must not alias any input.
 *   workspace    device memory of at least attn_bwd_workspace_size(B,H,S,D)
 *                bytes, 256-byte aligned, owned by the caller; its contents
 *                on entry do not matter and are garbage on return.
 * Every output is deterministic (no atomics).  Enqueues two kernels on
 * `stream`: dQ (one workgroup per 256-row query block), which also writes the
 * row statistics into the workspace, then dK/dV (one workgroup per 128-key
 * block), which reads them.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* dout, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes, int B, int H, int S,
             int D, float scale, int causal, attn_stream_t stream);

/* Phases of the backward, for attn_bwd_phases. */
enum attn_bwd_phase {
  ATTN_BWD_PRE = 1,   /* -LSE*log2(e), -Delta = -rowsum(dO * O) records into the workspace */
  ATTN_BWD_MAIN = 2,  /* dK, dV written (reads the workspace)                      */
  ATTN_BWD_DQ = 4,    /* dQ written; writes the same statistics as PRE             */
  ATTN_BWD_ALL = 7
};

/*
 * attn_bwd restricted to the phases set in `phases` (a nonzero subset of
 * ATTN_BWD_ALL), enqueued in the order PRE, DQ, MAIN; PRE is skipped when DQ
 * is requested, since DQ writes the same statistics.  MAIN reads the
 * statistics that PRE or DQ left in `workspace` (for the same o, lse, dout),
 * also from an earlier call.  For callers that time or schedule the phases
 * separately; arguments otherwise as attn_bwd.
 * phases == 0 or outside ATTN_BWD_ALL: ATTN_ERR_UNSUPPORTED.
 */
int attn_bwd_phases(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, int B, int H, int S,
                    int D, float scale, int causal, unsigned phases,
                    attn_stream_t stream);

/*
 * Backward that allocates nothing and takes no workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Computes exactly what attn_bwd
 * computes, with the same kernels, bit for bit; the workspace is a static
 * device array of attn_noalloc_scratch_bytes() (32 MiB) inside the library,
 * one per GPU, held until the process ends.  The call makes no hipMalloc,
 * hipFree or other allocating call (its first call on a device looks up that
 * device's copy of the array with hipGetSymbolAddress).
 *   Limit: attn_bwd_workspace_size(B, H, S, D) <= attn_noalloc_scratch_bytes(),
 *   i.e. B*H*ceil(S/64) <= 32768 (for example B*H = 32 heads up to S = 65536);
 *   larger shapes return ATTN_ERR_SCRATCH before any HIP call.
 *   Concurrency: every call on one GPU shares that GPU's array, so calls that
 *   overlap on one GPU (two streams, or two host threads) race and may return
 *   wrong gradients; serialise them, or use attn_bwd with a workspace each.
 *   The array keeps the last call's row statistics; nothing in it needs to
 *   start at zero.
 * Arguments (other than the absent workspace) and errors as attn_bwd.
 */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                     int B, int H, int S, int D, float scale, int causal,
                     attn_stream_t stream);

/* Size in bytes of attn_bwd_noalloc's static per-GPU workspace. */
size_t attn_noalloc_scratch_bytes(void);

/* Error reporting and versioning are conventions of this library (the pages
 * describe no interface): status codes instead of exceptions across the ABI. */

/* Static English description of a status code (never NULL). */
const char* attn_strerror(int status);

/* Raw hipError_t of the last ATTN_ERR_HIP returned on the calling thread. */
int attn_last_hip_error(void);

/* Library ABI version: major*10000 + minor*100 + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTN_H */
