/*
 * kda.h -- C ABI of the MI355X (gfx950) chunked forward of Kimi Delta Attention.
 *
 * The method (one value head, one sequence):
 *     S_t = (I - beta_t k_t k_t^T) diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 * computed in chunks of 64 tokens: an intra-chunk stage (per-dimension cumulative
 * gate, gated Aqk, the UT/WY inverse, w, u, qg, kg) and a serial inter-chunk state
 * scan that keeps h [K, V] in fp32:
 *     v' = u - w h,   o = scale * qg h + Aqk v',   h <- diag(exp2 G) h + kg^T v'.
 * Sources: "kernel-fun 0.2.0.dev1 -- kernel_fun/kda/_kernels/fwd_state.py",
 * module docstring (the chunk operands and the state scan) and host wrapper
 * (the call contract: bf16 operands, fp32 h0/ht [B, HV, K, V]); "KDA源码剖析之
 * FlashKDA（下）", the recurrence kernel's phases 3-6 (u = (v - k_decayed S) beta,
 * U = INV u, out = q_decayed S + Mqk U, S <- g_total S + k_restored^T U) and the
 * sequence-information section (varlen via cu_seqlens, one state per sequence).
 *
 * Conventions for every entry point below
 *   - Tensor pointers are DEVICE pointers to contiguous row-major memory; the
 *     caller owns every buffer.  The library never allocates, frees or
 *     synchronises.  Between calls it keeps only per-device caches (the
 *     compute-unit count, and the address of kda_fwd_no_alloc's static scratch),
 *     filled race-free on first use: every entry point is thread-safe and
 *     reentrant, except that kda_fwd_no_alloc calls overlapping in time on one
 *     device share that scratch (see there).
 *   - bf16 tensors are IEEE bfloat16 bit patterns (uint16).
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the null stream);
 *     calls return before the GPU work finishes.
 *   - Validation happens on the host before anything is launched.  On any error
 *     status nothing is launched and no output or workspace byte is touched.
 *   - A device-side check rejects cu_seqlens that is not non-decreasing from 0 to
 *     T; the outputs o and ht are then filled with NaN (loudly wrong), since the
 *     host cannot see device memory without synchronising.
 */
#ifndef KDA_MI355X_H
#define KDA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define KDA_OK                 0
#define KDA_ERR_INVALID_ARG   -1  /* null/misaligned pointer, bad size, HV % HQK != 0 ...  */
#define KDA_ERR_UNSUPPORTED   -2  /* K not in {64, 128}, V not a multiple of 16           */
#define KDA_ERR_WORKSPACE     -3  /* workspace NULL, misaligned or smaller than required  */
#define KDA_ERR_HIP           -4  /* a HIP launch failed; see kda_strerror                */
#define KDA_ERR_TOO_LARGE     -5  /* kda_fwd_no_alloc: the shapes need more scratch than
                                     KDA_NO_ALLOC_MAX_BYTES                                */

/* Chunk length of the chunked form (tokens per chunk) by default; see
 * kda_fwd_args.chunk for the 16-token variant. */
#define KDA_CHUNK 64

/* Option bits of kda_fwd_args.flags (FlashKDA's input and state variants,
 * "KDA源码剖析之FlashKDA（下）", parameter list of the forward entry point). */
#define KDA_FLAG_BETA_LOGITS  1u  /* beta holds raw logits; the kernel applies the sigmoid */
#define KDA_FLAG_STATE_BF16   2u  /* h0, ht and hc are bf16 instead of fp32                */
/* Option bit of kda_bwd_dhu_args.flags (with KDA_FLAG_STATE_BF16 for dht / dh0):
 * the per-chunk gradient checkpoints dhc are bf16, the checkpoint format of the
 * kernel-fun bwd_dhu page (host wrapper), instead of fp32. */
#define KDA_FLAG_CKPT_BF16    4u

typedef struct kda_fwd_args {
  /* Inputs (device, bf16 unless stated).
   *   q, k : [B, T, HQK, K]  keys/queries, expected L2-normalised over K by the caller
   *   v    : [B, T, HV,  V]
   *   g    : [B, T, HV,  K]  natural-log per-dimension decay, g <= 0; values
   *          below -10, -inf included, are taken as -10 (a decay of 4.5e-5
   *          instead of a smaller one: the outputs change by at most 4.5e-5 of the
   *          state it multiplies); so is a NaN with its sign bit set
   *   beta : [B, T, HV]      write strength in [0, 1] (already through a sigmoid),
   *          or its logit with KDA_FLAG_BETA_LOGITS
   *   h0   : [N, HV, K, V] initial state per sequence and value head, fp32 (bf16
   *          with KDA_FLAG_STATE_BF16), or NULL for a zero initial state.
   *   cu_seqlens : int64 [N + 1] on the device, or NULL.  NULL = fixed length:
   *          N = B sequences of T tokens.  Non-NULL = varlen: B must be 1, the N
   *          sequences are rows [cu[n], cu[n+1]) of the packed row, cu[0] = 0,
   *          cu[N] = T; each sequence starts from its own h0 and chunks restart at
   *          every sequence start (lengths need not be multiples of 64; empty
   *          sequences are allowed and return ht = h0).
   * Value head h reads q/k head h / (HV / HQK) (consecutive value heads share). */
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  float scale;                 /* usually K^-0.5                                      */
  const void* h0;
  const int64_t* cu_seqlens;
  int32_t B, T, HQK, HV, K, V; /* K in {64, 128}; V a positive multiple of 16         */
  int32_t N;                   /* number of sequences: == B (fixed) or len(cu) - 1    */
  /* Outputs (device, caller-allocated).
   *   o  : bf16 [B, T, HV, V]   every row of every sequence is written
   *   ht : [N, HV, K, V]   final state per sequence (state dtype), or NULL to skip
   * Alignment (else KDA_ERR_INVALID_ARG): q, k, v, g, h0, ht 16 bytes; o and
   * cu_seqlens 8 bytes; beta 2 bytes.  All tensors are dense, row-major.       */
  void* o;
  void* ht;
  /* Scratch (device, caller-allocated, 256-byte aligned, size from
   * kda_fwd_workspace_bytes).  Contents on entry do not matter. */
  void* workspace;
  size_t workspace_bytes;
  void* stream;                /* hipStream_t */
  /* Options; all-zero keeps the behaviour described above. */
  uint32_t flags;              /* KDA_FLAG_* bits; unknown bits are rejected          */
  /* Per-chunk states (kda_fwd / kda_fwd_inter), or NULL to skip them:
   *   hc : [C, HV, K, V] in the state dtype, the state *before* each chunk, chunks
   *        numbered sequence by sequence (sequence n's chunk j is chunk
   *        sum_{m<n} ceil(len_m / 64) + j; fixed length: n * ceil(T/64) + j).
   *        C must be at least that total: B * ceil(T/64) for fixed length; for
   *        varlen ceil(T/64) + N always suffices (rows past the total are not
   *        written).  Alignment 16 bytes (fp32) or 8 bytes (bf16).
   * The chunked backward pass needs these (kernel-fun fwd_state module docstring,
   * which keeps h per chunk for the backward). */
  void* hc;
  /* Segment length of the state scan in chunks (kda_fwd / kda_fwd_inter and the
   * workspace size), or 0 to let the library choose.  Each sequence is cut into
   * segments of this many chunks that are scanned in parallel and joined through
   * the scan's affine dependence on its start state; results do not depend on
   * it beyond rounding.  Must be >= 0. */
  int32_t seg_chunks;
  /* Chunk length of the chunked form: 64 (0 also means 64) or 16, the chunk length
   * of FlashKDA's recurrence kernel ("KDA源码剖析之FlashKDA（下）", kernel 2, template
   * parameter CHUNK = 16).  With 16 the state is updated every 16 tokens and the
   * intra-chunk terms (Aqk, the UT/WY inverse, w) span 16 tokens; o and ht equal
   * those of chunk 64 up to rounding.  hc is not available with 16
   * (KDA_ERR_UNSUPPORTED); the workspace size does not depend on it.  Other values:
   * KDA_ERR_UNSUPPORTED. */
  int32_t chunk;
} kda_fwd_args;

/* Largest workspace kda_fwd_no_alloc can use: the size of the library's static
 * per-device scratch buffer. */
#define KDA_NO_ALLOC_MAX_BYTES ((size_t)128 << 20)

/* Workspace size for these arguments (host only, launches nothing).  Only the
 * shape fields (B, T, HQK, HV, K, V, N, whether cu_seqlens is NULL) and seg_chunks
 * are read.  With seg_chunks == 0 the size follows the state scan the library picks
 * for the compute-unit count of the device current on the calling thread, so a
 * workspace sized on one device kind fits calls made with that device current.
 * Returns KDA_OK and *bytes, or an error status. */
int kda_fwd_workspace_bytes(const kda_fwd_args* a, size_t* bytes);

/* The state scan these arguments select (host only, launches nothing; reads the same
 * fields as kda_fwd_workspace_bytes plus seg_chunks).  On KDA_OK, *seg_chunks is 0
 * for the 16-column serial scan, else the segment length in chunks of the
 * 64-column scan (a value >= every sequence's chunk count means one segment per
 * sequence).  The choice depends on the device's compute-unit count: with more
 * 64-column workgroups than compute units one segment per sequence; else, for
 * sequences of 96 chunks or more (the mean for varlen), 2 to 8 segments so that
 * the full pass fills the device in one round; else the serial scan when its
 * workgroups fill at least half the device or sequences are shorter than 32
 * chunks, and segments of max(4, ceil(chunks / 8)) otherwise. */
int kda_fwd_scan_plan(const kda_fwd_args* a, int32_t* seg_chunks);

/* The whole chunked forward: o (and ht) from q, k, v, g, beta, h0 (kernel-fun
 * docstring; FlashKDA recurrence phases 3-6).  Equivalent to kda_fwd_intra
 * followed by kda_fwd_inter on the same stream. */
int kda_fwd(const kda_fwd_args* a);

/* kda_fwd without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same kernels and results as kda_fwd; a->workspace and
 * a->workspace_bytes are ignored.  The scratch is a static device array of
 * KDA_NO_ALLOC_MAX_BYTES that the library holds on every device it runs on until the
 * process ends; its address is looked up on the first call on each device.  The call
 * allocates nothing: shapes whose kda_fwd_workspace_bytes exceeds
 * KDA_NO_ALLOC_MAX_BYTES are rejected with KDA_ERR_TOO_LARGE before any launch (at
 * K = V = 128 about 2,000 (chunk, value head) pairs fit, e.g. 4,096 tokens x 32
 * heads).  Every call on one device shares that device's buffer: calls that overlap
 * in time on one device (different streams, or threads) race and must not be made;
 * calls in stream order are safe, since each call rewrites every byte it reads (the
 * work counter and chunk tables are reset by the call's first kernel). */
int kda_fwd_no_alloc(const kda_fwd_args* a);

/* Intra-chunk stage only (per-dimension gate cumsum, gated Aqk, Akk and its
 * UT/WY inverse, w, qg, kg; kernel-fun docstring): fills the workspace from
 * q, k, g, beta (and the varlen chunk table from cu_seqlens).  o, ht, v, h0 are
 * not read.  Exposed so the two stages can be timed separately. */
int kda_fwd_intra(const kda_fwd_args* a);

/* Inter-chunk state scan only (kernel-fun docstring: v' = u - w h, o = scale qg h
 * + Aqk v', h <- diag(exp2 G) h + kg^T v'): reads the workspace written by
 * kda_fwd_intra with the same arguments, plus v and h0; writes o and ht. */
int kda_fwd_inter(const kda_fwd_args* a);

/* Debug view of the intra-stage results (after kda_fwd_intra with the same
 * arguments), unpacked from the workspace's internal layout into plain tensors.
 * Any output pointer may be NULL to skip it.
 *   qg   : bf16 [B, T, HV, K]   scale * q * exp(Gam)   (Gam = in-chunk gate cumsum)
 *   w    : bf16 [B, T, HV, K]   Tm diag(beta) (k * exp(Gam))
 *   kg   : bf16 [B, T, HV, K]   k * exp(Gam_last - Gam)
 *   aqk  : bf16 [B, T, HV, 64]  row i of the chunk's Aqk (columns = chunk rows)
 *   tmb  : bf16 [B, T, HV, 64]  row i of Tm diag(beta), Tm = (I + Akk)^-1
 *   alpha: fp32 [B, T, HV, K]   exp(Gam_last) of the row's chunk, on every row
 * Rows of each sequence are written; other memory is untouched. */
int kda_debug_unpack(const kda_fwd_args* a, void* qg, void* w, void* kg, void* aqk,
                     void* tmb, float* alpha);

/* ------------------------------------------------------------------------
 * Reverse state scan of the chunked backward pass ("kernel-fun 0.2.0.dev1 --
 * kernel_fun/kda/_kernels/bwd_dhu.py", module docstring and host wrapper).  For a
 * loss with gradient do of o and dht of the final state, per sequence and value
 * head, dh starts at dht (or 0) and walks the chunks newest first:
 *     dhc[c] = dh                                   (gradient of the state after chunk c)
 *     dv2    = kg dh + dv                            (per token row of the chunk)
 *     dh    <- diag(exp2 gd) dh + scale qg^T do - w^T dv2,   gd = g2 at the chunk's last row
 * and dh0 = dh after the sequence's first chunk.  Chunks are 64 tokens and restart
 * at every sequence start, as in the forward.  Conventions as for kda_fwd_args.
 */
typedef struct kda_bwd_dhu_args {
  /* Inputs (device).  The forward's chunk operands, recomputed by the caller:
   *   qg  : bf16 [B, T, HV, K]  q * exp2(g2)                (no scale folded in)
   *   kg  : bf16 [B, T, HV, K]  k * exp2(g2_last - g2)      (g2_last: the chunk's last valid row)
   *   w   : bf16 [B, T, HV, K]  Tm diag(beta) (k * exp2(g2)), the forward's w
   *   g2  : fp32 [B, T, HV, K]  chunk-local inclusive cumsum of g in log2 units
   *         (G / ln 2); only each chunk's last valid row is read
   *   dout: bf16 [B, T, HV, V]  gradient of o
   *   dv  : bf16 [B, T, HV, V]  the part of the gradient of v' that does not pass
   *         through the state (Aqk^T do per chunk), or NULL for zero
   *   dht : [N, HV, K, V] gradient of the final state (fp32, bf16 with
   *         KDA_FLAG_STATE_BF16), or NULL for zero
   *   cu_seqlens, B, T, HV, K, V, N: as in kda_fwd_args (K in {64, 128}, V a
   *         positive multiple of 16; varlen: B == 1). */
  const void* qg;
  const void* kg;
  const void* w;
  const float* g2;
  const void* dout;
  const void* dv;
  const void* dht;
  float scale;                 /* usually K^-0.5                                      */
  const int64_t* cu_seqlens;
  int32_t B, T, HV, K, V, N;
  /* Outputs (device, caller-allocated).
   *   dv2 : bf16 [B, T, HV, V]  every row of every sequence is written
   *   dh0 : [N, HV, K, V] (dht's dtype), or NULL to skip
   *   dhc : [C, HV, K, V] fp32 (bf16 with KDA_FLAG_CKPT_BF16), chunks numbered and
   *         C sized as hc of kda_fwd_args, or NULL to skip
   * Alignment (else KDA_ERR_INVALID_ARG): qg, kg, w, g2, dht, dh0, dhc 16 bytes;
   * dout, dv, dv2 and cu_seqlens 8 bytes. */
  void* dv2;
  void* dh0;
  void* dhc;
  /* Scratch (device, 256-byte aligned, size from kda_bwd_dhu_workspace_bytes: for varlen
   * the chunk and segment tables and the sequences' longest-first order, and, when a
   * sequence has several segments, each segment's b (fp32 K x V) and M (bf16 K x K) per
   * value head; all written by the call itself.  Zero bytes, so NULL is allowed, for
   * fixed length with one segment per sequence). */
  void* workspace;
  size_t workspace_bytes;
  void* stream;                /* hipStream_t */
  uint32_t flags;              /* KDA_FLAG_STATE_BF16 | KDA_FLAG_CKPT_BF16; others rejected */
  /* Segment length of the scan in chunks, or 0 to let the library choose (the forward's
   * rule, kda_fwd_scan_plan).  As in the forward, sequences cut into segments are scanned in
   * parallel by 64-column workgroups and joined through the recursion's affine dependence on
   * dh (a state pass computes each segment's hand-on b and transition M first); results do
   * not depend on it beyond rounding.  Must be >= 0. */
  int32_t seg_chunks;
} kda_bwd_dhu_args;

/* Workspace size for these arguments (host only; reads the shape fields, whether
 * cu_seqlens is NULL and seg_chunks; with seg_chunks == 0 the plan follows the current
 * device's compute-unit count, as for the forward). */
int kda_bwd_dhu_workspace_bytes(const kda_bwd_dhu_args* a, size_t* bytes);

/* The reverse state scan: dv2, dh0 and dhc from qg, kg, w, g2, dout, dv, dht.
 * Rejected cu_seqlens (checked on the device) fill dv2 and dh0 with NaN. */
int kda_bwd_dhu(const kda_bwd_dhu_args* a);

/* Static text for a status code, or for the last HIP error seen by this thread
 * when status == KDA_ERR_HIP. */
const char* kda_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* KDA_MI355X_H */
