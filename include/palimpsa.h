/*
 * palimpsa.h - C ABI of libpalimpsa.so, the MI355X (gfx950) implementation
 * of the Palimpsa dual-state recurrence.
 *
 * The operation ("Learning to Remember, Learn, and Forget in Attention-Based
 * Models", slides frames "The attention state is an online regression
 * model", "Forgetting discounts evidence and restores the prior" and
 * "Palimpsa updates content and importance together", Eqs. (1)-(2), (5), (9)):
 * for every sequence b and head h, with value channel i < dv and key
 * channel j < dk,
 *
 *     alpha_t    = exp(-A[h] * dt[b,t,h])                       (gate, in (0, 1])
 *     I_t[i,j]   = alpha_t I_{t-1}[i,j] + (1 - alpha_t) I_prior[h]
 *                  + beta[b,t,h,i] * k[b,t,h,j]^2                (importance)
 *     mu_t[i,j]  = alpha_t (I_{t-1}[i,j] / I_t[i,j]) mu_{t-1}[i,j]
 *                  + beta[b,t,h,i] v[b,t,h,i] k[b,t,h,j] / I_t[i,j]   (content)
 *     y[b,t,h,i] = sum_j mu_t[i,j] q[b,t,h,j]                   (readout, after the write)
 *
 * The chunked forward evaluates it in the natural parameters M = I . mu and
 * I (slides frame "Natural parameters expose two affine scans", App. A.12),
 * which is the same function up to float32 rounding.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers, owned by the caller, contiguous and
 *    row-major in the layouts stated per argument.  Pointers the kernels read
 *    or write with 128-bit accesses must be 16-byte aligned: q, k, v, beta and
 *    the state arrays of palimpsa_fwd_chunked, and mu, I of palimpsa_step.
 *    Every other pointer needs the natural alignment of its element type.
 *  - in_dtype applies to q, k, v, beta and dt; out_dtype to y (gy_dtype to the
 *    backward's gy).  They are int parameters holding a palimpsa_dtype value,
 *    so that any int, valid or not, reaches the validation (which rejects
 *    the others) as a defined value.  A, I_prior and every state array are
 *    float32.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL means the default
 *    stream) and runs asynchronously; the caller synchronises.
 *  - The library allocates no device memory and keeps no per-call state;
 *    scratch, where a call uses any, is a caller-owned workspace argument.
 *  - Every argument is checked on the host before anything is launched; an
 *    invalid call returns an error code and launches nothing.  No C++
 *    exception crosses this interface.
 *  - Data preconditions that are NOT checked (they live in device memory):
 *    A >= 0 and finite, I_prior > 0, beta >= 0, dt >= 0, I0 > 0, all inputs
 *    finite.  Violations give unspecified values, never a fault.  (The Python
 *    binding's check_params tests them on request.)
 *  - Supported head sizes: dk in {32, 64, 128}; dv any multiple of 16 from
 *    16 to 1024 (so the value expansion dv = 2 dk of the pages' model is
 *    covered).  The chunked forward and the decode step also take heads as
 *    wide as the model (the pages' recurrent-kernel measurement, slides
 *    frame 22 / Fig. 7): dk in {256, 512, 1024, 2048} with dv a multiple of 16
 *    up to 4096 (up to 1024 at dk = 256), per-head prior, flags 0, and no
 *    time split for dk >= 512.  The other paths' limits are stated at their
 *    declarations.
 *  - Options (`flags`, a bit mask of palimpsa_flags) of the exact forward,
 *    the decode step and the backward:
 *      PALIMPSA_VSTAR            v holds v* = beta . v, the write itself (the
 *                                slides' frame on the Mamba2 limit makes v*
 *                                the layer's input); beta still scales k^2 in
 *                                the importance.  The backward's gv is then
 *                                dL/dv*, and gbeta has only the importance term.
 *      PALIMPSA_PRIOR_PER_ENTRY  I_prior is [H, dv, dk] float32, one prior
 *                                precision per state entry (the reading notes'
 *                                symbol table allows a prior of the state's
 *                                shape); 16-byte aligned.  The prior term is
 *                                (1 - alpha_t) I_prior[h, i, j]; the default
 *                                start state is I0 = I_prior entry by entry;
 *                                the backward's gIp is [H, dv, dk].
 *    Two more bits pair one training forward with its backward, so that the
 *    backward need not recompute the states (see palimpsa_bwd):
 *      PALIMPSA_SAVE_CHECKPOINTS  (forward only) also store the backward's
 *                                state checkpoints into `workspace`, which is
 *                                then a backward workspace.
 *      PALIMPSA_CHECKPOINTS_SAVED (backward only) the workspace already holds
 *                                them; the backward skips its first pass.
 *    Unknown bits, and a bit on an entry point it does not apply to, are
 *    PALIMPSA_ERR_INVALID_ARG.
 */
#ifndef PALIMPSA_H
#define PALIMPSA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PALIMPSA_OK = 0,
    PALIMPSA_ERR_INVALID_ARG = 1,  /* null pointer, negative or zero size, bad enum */
    PALIMPSA_ERR_UNSUPPORTED = 2,  /* valid but not implemented (head size, dtype pair) */
    PALIMPSA_ERR_ALIGNMENT = 3,    /* a tensor pointer breaks the alignment rule above */
    PALIMPSA_ERR_HIP = 4,          /* the HIP runtime reported an error at launch */
    PALIMPSA_ERR_SCRATCH_LIMIT = 5 /* palimpsa_fwd_chunked_noalloc: the call would need more
                                      scratch than the library's fixed buffer holds */
} palimpsa_status;

typedef enum {
    PALIMPSA_F32 = 0,
    PALIMPSA_BF16 = 1
} palimpsa_dtype;

typedef enum {
    PALIMPSA_VSTAR = 1,
    PALIMPSA_PRIOR_PER_ENTRY = 2,
    PALIMPSA_SAVE_CHECKPOINTS = 4,
    PALIMPSA_CHECKPOINTS_SAVED = 8
} palimpsa_flags;

/*
 * Chunked forward over a whole sequence (training / prefill).
 *
 *   q, k      [B, T, H, dk]  in_dtype
 *   v, beta   [B, T, H, dv]  in_dtype
 *   dt        [B, T, H]      in_dtype
 *   A         [H]            float32, per-head decay rate
 *   I_prior   [H]            float32, per-head prior precision
 *             ([H, dv, dk] with PALIMPSA_PRIOR_PER_ENTRY)
 *   mu0, I0   [B, H, dv, dk] float32 initial state; both NULL means
 *                            mu0 = 0 and I0 = I_prior (one NULL alone is an error)
 *   y         [B, T, H, dv]  out_dtype, every token's readout
 *   muT, IT   [B, H, dv, dk] float32 final state; both NULL skips writing it
 *                            (one NULL alone is an error).  muT may alias mu0
 *                            and IT may alias I0 (in-place resume).
 *   chunk     the most tokens to stage per step through on-chip memory, one
 *             of {8, 16, 32, 64, 128}, or 0 for the library's choice (the
 *             largest of 16, 32, 64 whose staging buffers let three
 *             workgroups share a CU when the grid is large enough to need it,
 *             else the largest that fits the device's LDS).  A nonzero chunk
 *             caps that choice (8 is run as 16).  A performance hint only: the
 *             results are bit-identical for every chunk.
 *   segments  time segments (0..64).  1: one pass over the sequence.  >= 2:
 *             cut T into that many segments (lengths rounded up to multiples
 *             of 64 tokens, so fewer may result) that run side by side: a
 *             summary pass computes each segment's affine map from a zero
 *             state (M_loc, Ibar_loc and the decay product, the composable
 *             form of the natural-parameter scans, slides frame "Natural
 *             parameters expose two affine scans"), then a replay pass starts
 *             every segment from the composition of the earlier maps and reads
 *             out.  0: the library decides (it splits only when the B*H*dv/16
 *             workgroups would be fewer than two per CU, into whole rounds of
 *             three workgroups per CU, up to 32 segments of at least 256
 *             tokens, within the no-allocation scratch size).  Results of a
 *             split match the single pass up to float32 rounding.
 *   workspace, workspace_bytes
 *             device scratch for the segment summaries and a copy of the
 *             start state (so that an in-place resume stays correct under a
 *             split), owned by the caller, 16-byte aligned;
 *             palimpsa_fwd_workspace_size() gives the size.
 *             NULL / 0 is valid: with segments == 0 the forward then runs in
 *             one pass; an explicit segments >= 2 without enough workspace is
 *             PALIMPSA_ERR_INVALID_ARG.  Contents are overwritten; calls that
 *             share a workspace must not overlap.
 *             Heads of dk >= 512 (dv a multiple of 64, T >= 1, and at least
 *             one workgroup of 64 value rows x one column slice per CU) use
 *             it for the row-parallel form: per-token records of the column
 *             operands (14 bytes per token and key column) and each column
 *             slice's partial readout (4 bytes per output element and slice;
 *             2 slices at dk = 512 and 1024, 4 at 2048);
 *             palimpsa_fwd_workspace_size() reports that size.  Without it (NULL, or fewer bytes) such heads run the
 *             column-parallel kernel: the final state is the same bits and y
 *             differs only in the float32 order of its sum over key columns.
 *   flags     palimpsa_flags bits (see above), or 0.
 *
 * With PALIMPSA_SAVE_CHECKPOINTS (the training forward) the workspace is a
 * backward workspace of at least palimpsa_bwd_workspace_size(B, T, H, dk, dv,
 * flags) bytes (else PALIMPSA_ERR_INVALID_ARG); the forward runs in one pass
 * (segments must be 0 or 1, chunk 0 or 16, dk <= 128, dv <= 1024, else
 * PALIMPSA_ERR_UNSUPPORTED) and also stores the state before every 16th token
 * there, bit-identical to what palimpsa_bwd would recompute.  A backward called
 * on the same inputs, flags (PALIMPSA_CHECKPOINTS_SAVED in place of
 * PALIMPSA_SAVE_CHECKPOINTS) and workspace then reuses them.
 *
 * T == 0 is valid: y is empty and the state is copied through (or, with both
 * mu0 and I0 NULL, set to mu = 0, I = I_prior); the per-token pointers q, k,
 * v, beta, dt and y are then not read and may be NULL.  B, H >= 1.
 * bf16 inputs are read exactly; bf16 outputs are rounded to nearest even.
 */
palimpsa_status palimpsa_fwd_chunked(const void *q, const void *k, const void *v,
                                     const void *beta, const void *dt,
                                     const float *A, const float *I_prior,
                                     const float *mu0, const float *I0,
                                     void *y, float *muT, float *IT,
                                     int B, int T, int H, int dk, int dv, int chunk,
                                     int segments, int in_dtype,
                                     int out_dtype, int flags, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * palimpsa_fwd_chunked for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same operation, arguments and results as
 * palimpsa_fwd_chunked with a large enough workspace, but it takes none.  A
 * time split keeps its segment summaries and its copy of the start state in a
 * fixed scratch array inside the library instead, palimpsa_noalloc_scratch_bytes()
 * bytes (64 MiB) on each GPU the library runs on, held until the process ends.
 * The call allocates nothing.
 *
 *   flags     as palimpsa_fwd_chunked, except PALIMPSA_SAVE_CHECKPOINTS
 *             (whose workspace is a backward's): PALIMPSA_ERR_INVALID_ARG
 *
 * A call whose split (the library's own choice with segments == 0, or the
 * one asked for) would need more scratch than that returns
 * PALIMPSA_ERR_SCRATCH_LIMIT and launches nothing; every split the library
 * chooses by itself fits (its choice is capped to this size).
 * Heads of dk >= 512 run the column-parallel kernel here (the row-parallel
 * form's workspace is gigabytes): results as palimpsa_fwd_chunked without a
 * workspace.
 * Calls on one GPU share its scratch array: calls that can overlap on one GPU
 * (other streams, other threads) race and must be ordered by the caller.
 * The first call on a device looks the array's address up (with that device
 * current); later calls reuse it.
 */
palimpsa_status palimpsa_fwd_chunked_noalloc(const void *q, const void *k, const void *v,
                                             const void *beta, const void *dt,
                                             const float *A, const float *I_prior,
                                             const float *mu0, const float *I0,
                                             void *y, float *muT, float *IT,
                                             int B, int T, int H, int dk, int dv, int chunk,
                                             int segments, int in_dtype,
                                             int out_dtype, int flags, void *stream);

/* Bytes of the fixed scratch array palimpsa_fwd_chunked_noalloc uses per GPU. */
size_t palimpsa_noalloc_scratch_bytes(void);

/*
 * Bytes of workspace palimpsa_fwd_chunked needs for the split it would choose
 * for these sizes and `segments` on the current device (0: no split, no
 * workspace), or, for dk >= 512, for the row-parallel form (0 where that
 * form is not taken; `segments` is then not used).  Returns 0 for sizes the
 * forward would reject.
 */
size_t palimpsa_fwd_workspace_size(int B, int T, int H, int dk, int dv, int segments);

/*
 * Frozen-importance forward: the Mamba2 limit of the recurrence, in which the
 * importance stays at I_prior (slides frame "The Mamba2 limit enables a
 * gradual model upgrade"; reading notes section 2.8):
 *
 *     mu_t = alpha_t mu_{t-1} + (beta_t . v_t / I_prior[h]) (x) k_t,   y_t = mu_t q_t
 *
 * It is the recurrence of the "without metaplasticity" model that a Palimpsa
 * layer upgrades, and the exact form's limit for small excess importance.
 * Its chunked form is dense, so it runs on the matrix cores (bf16 operands,
 * fp32 accumulation, fp32 state).
 *
 *   q, k      [B, T, H, dk]  bf16 (in_dtype must be PALIMPSA_BF16)
 *   v, beta   [B, T, H, dv]  bf16; beta NULL means v already holds beta . v
 *             (the reparameterised write v* of the same frame)
 *   dt        [B, T, H]      bf16
 *   A, I_prior [H]           float32
 *   mu0       [B, H, dv, dk] float32 initial mean, or NULL for 0
 *   y         [B, T, H, dv]  out_dtype
 *   muT       [B, H, dv, dk] float32 final mean, or NULL to skip
 *
 * dk in {64, 128}, dv a multiple of 64 up to 1024; other sizes or fp32
 * inputs return PALIMPSA_ERR_UNSUPPORTED.  (A prior per state entry would
 * make the write per entry instead of an outer product, so this path takes
 * the per-head prior only.)
 * q, k, v, beta, mu0, muT and y must be 16-byte aligned.  Rounding: operands
 * of the products are bf16, so y carries about 2^-8 relative error.
 */
palimpsa_status palimpsa_fwd_frozen(const void *q, const void *k, const void *v,
                                    const void *beta, const void *dt,
                                    const float *A, const float *I_prior, const float *mu0,
                                    void *y, float *muT, int B, int T, int H, int dk, int dv,
                                    int in_dtype, int out_dtype,
                                    void *stream);

/*
 * One decode token (recurrent inference): the recurrence above for a single
 * t, applied in place to a state held as (mu, I).
 *
 *   q, k      [B, H, dk]     in_dtype
 *   v, beta   [B, H, dv]     in_dtype
 *   dt        [B, H]         in_dtype
 *   A, I_prior [H]           float32 (I_prior [H, dv, dk] with PALIMPSA_PRIOR_PER_ENTRY)
 *   mu, I     [B, H, dv, dk] float32, read and overwritten with the new state
 *   y         [B, H, dv]     out_dtype
 *   flags     palimpsa_flags bits, or 0
 */
palimpsa_status palimpsa_step(const void *q, const void *k, const void *v,
                              const void *beta, const void *dt,
                              const float *A, const float *I_prior,
                              float *mu, float *I, void *y,
                              int B, int H, int dk, int dv,
                              int in_dtype, int out_dtype, int flags,
                              void *stream);

/*
 * Backward of palimpsa_fwd_chunked (training).  The pages train through the
 * recurrence but print no backward; this is the exact reverse-mode
 * derivative (vector-Jacobian product) of the forward above for the scalar
 *
 *     L = sum(gy . y) + sum(gmuT . muT) + sum(gIT . IT),
 *
 * taken through the natural-parameter scans of the slides' frame "Natural
 * parameters expose two affine scans" (App. A.12) and the gate of Eq. (9)
 * (alpha = exp(-A dt), c = (1 - alpha) I_prior).  It recomputes the forward
 * states itself (checkpoints every 16 tokens in the workspace), so it takes
 * the forward's inputs, not its outputs.
 *
 * Inputs (device pointers, layouts and dtypes as palimpsa_fwd_chunked):
 *   q, k, v, beta, dt, A, I_prior, mu0, I0   the forward's inputs (mu0 and I0
 *             both NULL: the default start state mu0 = 0, I0 = I_prior)
 *   gy        [B, T, H, dv]  gy_dtype   dL/dy
 *   gmuT, gIT [B, H, dv, dk] float32    dL/dmuT, dL/dIT; each may be NULL (zero)
 * Outputs (float32, overwritten):
 *   gq, gk    [B, T, H, dk]     gv, gbeta [B, T, H, dv]     gdt [B, T, H]
 *   gA, gIp   [H]   summed over the batch; with the default start state gIp
 *             includes the share of I0 = I_prior
 *   gmu0, gI0 [B, H, dv, dk]  gradient of the start state, or NULL to skip
 *             (with the default start state: the gradient at mu0 = 0, I0 = I_prior)
 *   workspace at least palimpsa_bwd_workspace_size(B, T, H, dk, dv) bytes,
 *             16-byte aligned, caller-owned; contents on entry are ignored
 *
 * flags: palimpsa_flags bits (the options change gv, gbeta and the shape of
 * gIp as stated above); the workspace size depends on them.  With
 * PALIMPSA_CHECKPOINTS_SAVED the workspace must hold the checkpoints that a
 * palimpsa_fwd_chunked call with PALIMPSA_SAVE_CHECKPOINTS stored for the same
 * q, k, v, beta, dt, A, I_prior, mu0, I0, sizes and option bits, and nothing
 * may have written to it since; the backward then skips recomputing them
 * (results are bit-identical to the backward without the bit).  The library
 * cannot check this pairing: a workspace that does not hold them gives wrong
 * gradients, not an error.  The backward leaves the checkpoints in place.
 *
 * dk in {32, 64, 128}, dv a multiple of 16 up to 1024 (else
 * PALIMPSA_ERR_UNSUPPORTED).  q, k, v, beta,
 * gy, the state arrays, gq, gk and the workspace must be 16-byte aligned;
 * the other pointers naturally aligned.  At T = 0 the per-token pointers may
 * be NULL.  Launches are asynchronous on `stream`; calls that share a
 * workspace must not overlap.  Arithmetic is float32; results are
 * deterministic (no atomics).
 */
palimpsa_status palimpsa_bwd(const void *q, const void *k, const void *v, const void *beta,
                             const void *dt, const float *A, const float *I_prior,
                             const float *mu0, const float *I0,
                             const void *gy, const float *gmuT, const float *gIT,
                             float *gq, float *gk, float *gv, float *gbeta, float *gdt,
                             float *gA, float *gIp, float *gmu0, float *gI0,
                             int B, int T, int H, int dk, int dv,
                             int in_dtype, int gy_dtype, int flags,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of workspace palimpsa_bwd needs: the checkpoints (8 B per state
 * entry every 16 tokens: B H ceil(T/16) dv dk 8 bytes) plus the per-row-block
 * partials of gq, gk (dv/16 x B T H x 2 dk x 4 bytes) and small sums; with
 * PALIMPSA_PRIOR_PER_ENTRY also each sequence's gIp (B H dv dk x 4 bytes).
 * Returns 0 for sizes or flags palimpsa_bwd would reject.  flags may carry
 * either checkpoint bit; only PALIMPSA_PRIOR_PER_ENTRY changes the size.
 */
size_t palimpsa_bwd_workspace_size(int B, int T, int H, int dk, int dv, int flags);

/*
 * Backward of palimpsa_fwd_frozen (training the frozen-importance model that a
 * Palimpsa layer upgrades, slides frame "The Mamba2 limit enables a gradual
 * model upgrade").  The exact reverse-mode derivative of
 *
 *     mu_t = alpha_t mu_{t-1} + (w_t / I_prior[h]) (x) k_t,   y_t = mu_t q_t,
 *     w_t = beta_t . v_t (or v*_t when beta is NULL),  alpha_t = exp(-A dt_t),
 *
 * for L = sum(gy . y) + sum(gmuT . muT), from the forward's inputs (it
 * recomputes the states itself).  Two paths, chosen by the inputs:
 *   - bf16 inputs with dk in {64, 128} and dv in {64, 128, 256}: the chunked form on the matrix
 *     cores (64-token chunks; per chunk each gradient is one product with the
 *     chunk's boundary state or adjoint and one causal product inside the
 *     chunk).  Operands are bf16 as in palimpsa_fwd_frozen, accumulation fp32:
 *     gradients carry about 2^-8 relative error, and the batch sums gA and
 *     gIp that much of the sum of their terms' magnitudes;
 *   - otherwise (float32 inputs, dk = 32, other dv): float32 throughout, the
 *     states recomputed from checkpoints every 16 tokens.
 *
 * Inputs (device pointers, layouts as palimpsa_fwd_chunked):
 *   q, k      [B, T, H, dk]  in_dtype
 *   v, beta   [B, T, H, dv]  in_dtype; beta NULL: v holds the write v*
 *   dt        [B, T, H]      in_dtype
 *   A, I_prior [H]           float32 (per-head prior only)
 *   mu0       [B, H, dv, dk] float32 start mean, or NULL for 0
 *   gy        [B, T, H, dv]  gy_dtype   dL/dy
 *   gmuT      [B, H, dv, dk] float32    dL/dmuT, or NULL (zero)
 * Outputs (float32, overwritten):
 *   gq, gk    [B, T, H, dk]     gv [B, T, H, dv] (dL/dv*, with beta NULL)
 *   gbeta     [B, T, H, dv]     required with beta, not written without it
 *   gdt       [B, T, H]
 *   gA, gIp   [H]   summed over the batch
 *   gmu0      [B, H, dv, dk]    dL/dmu0 (at mu0 = 0 when mu0 is NULL), or NULL
 *   workspace at least palimpsa_bwd_workspace_size(B, T, H, dk, dv, 0) bytes,
 *             16-byte aligned, caller-owned; contents on entry are ignored
 *
 * dk in {32, 64, 128}, dv a multiple of 16 up to 1024 (else
 * PALIMPSA_ERR_UNSUPPORTED).  Alignment, T = 0, streams and determinism as
 * palimpsa_bwd.
 */
palimpsa_status palimpsa_bwd_frozen(const void *q, const void *k, const void *v, const void *beta,
                                    const void *dt, const float *A, const float *I_prior, const float *mu0,
                                    const void *gy, const float *gmuT,
                                    float *gq, float *gk, float *gv, float *gbeta, float *gdt,
                                    float *gA, float *gIp, float *gmu0,
                                    int B, int T, int H, int dk, int dv,
                                    int in_dtype, int gy_dtype,
                                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Forward with limited cross-key precision: block-diagonal P (the slides'
 * closing question on limited cross-key correlations).  Each value row runs
 * the full Gaussian update of the slides' backup frame "dropping precision
 * correlations changes the mean" (App. A.3-A.5),
 *
 *     P_t  = alpha_t P_{t-1} + (1 - alpha_t) I_prior[h] Id + beta_t[i] k_t k_t^T
 *     mu_t = P_t^{-1} [alpha_t P_{t-1} mu_{t-1} + beta_t[i] v_t[i] k_t],   y_t[i] = mu_t q_t
 *
 * with P kept block-diagonal along the key axis (blocks of `block` adjacent
 * key channels; the entries between blocks are dropped at every token, as
 * Eq. (5) drops every off-diagonal entry).  block == 1 is palimpsa_fwd_chunked;
 * this entry point implements block == 2 and block == 4.
 *
 *   q, k, v, beta, dt, A, I_prior, y   as palimpsa_fwd_chunked (per-head prior)
 *   mu0       [B, H, dv, dk] float32 initial mean, and
 *   P0        [B, H, dv, dk/block, block, block] float32 initial precision
 *             blocks (symmetric positive definite; only the upper triangle is
 *             read); both NULL: mu0 = 0, P0 = I_prior Id
 *   muT, PT   the final state in the same layouts (PT written in full,
 *             symmetric), or both NULL to skip
 *   flags     0, or PALIMPSA_SAVE_CHECKPOINTS (the training forward): also
 *             store the backward's checkpoints in workspace, which must then
 *             be the workspace of a following palimpsa_bwd_blockdiag call
 *             (palimpsa_bwd_blockdiag_workspace_size(B, T, H, dk, dv, block)
 *             bytes, 16-byte aligned) that passes PALIMPSA_CHECKPOINTS_SAVED;
 *             without the flag workspace is not read and may be NULL
 *
 * block == 2 with dk in {32, 64, 128}, or block == 4 with dk in {64, 128}; dv a
 * multiple of 16 up to 1024 (else PALIMPSA_ERR_UNSUPPORTED).  q, k, v, beta,
 * P0 and PT must be 16-byte aligned.  Arithmetic float32: each 2x2 block is
 * solved with a reciprocal of its determinant, each 4x4 block by Cholesky
 * (v_rsq_f32 for the diagonal); T == 0 copies the state through.
 */
palimpsa_status palimpsa_fwd_blockdiag(const void *q, const void *k, const void *v, const void *beta,
                                       const void *dt, const float *A, const float *I_prior,
                                       const float *mu0, const float *P0, void *y, float *muT, float *PT,
                                       int B, int T, int H, int dk, int dv, int block,
                                       int in_dtype, int out_dtype, int flags,
                                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode token of the block-diagonal-precision recurrence (2x2 or 4x4 blocks),
 * in place on the state (recurrent inference for the path above): per value
 * row i and key block (2j, 2j+1), the block's natural parameter h = P mu is
 * carried through the token as palimpsa_fwd_blockdiag carries it,
 *
 *     P'  = alpha P + (1 - alpha) I_prior[h] Id + beta[i] k k^T,
 *     h'  = alpha P mu + beta[i] v[i] k,   mu' = P'^{-1} h',   y[i] = sum_j mu' . q
 *
 *   q, k      [B, H, dk]     in_dtype
 *   v, beta   [B, H, dv]     in_dtype
 *   dt        [B, H]         in_dtype
 *   A, I_prior [H]           float32
 *   mu        [B, H, dv, dk] float32, read and overwritten
 *   P         [B, H, dv, dk/block, block, block] float32 precision blocks, read
 *             (upper triangle) and overwritten (in full, symmetric)
 *   y         [B, H, dv]     out_dtype
 *
 * block == 2 with dk in {32, 64, 128}, or block == 4 with dk in {64, 128}; dv a
 * multiple of 16 up to 1024 (else PALIMPSA_ERR_UNSUPPORTED).  mu and P must be
 * 16-byte aligned.  A 2x2 block is solved with a float32 division by its
 * determinant, a 4x4 block by Cholesky, so the step's results match
 * palimpsa_fwd_blockdiag over the same token up to float32 rounding.
 */
palimpsa_status palimpsa_step_blockdiag(const void *q, const void *k, const void *v, const void *beta,
                                        const void *dt, const float *A, const float *I_prior, float *mu, float *P,
                                        void *y, int B, int H, int dk, int dv, int block,
                                        int in_dtype, int out_dtype, void *stream);

/*
 * Bytes of workspace palimpsa_bwd_blockdiag needs for these sizes (0 for
 * sizes or a block it does not support).
 */
size_t palimpsa_bwd_blockdiag_workspace_size(int B, int T, int H, int dk, int dv, int block);

/*
 * Reverse-mode derivative of palimpsa_fwd_blockdiag (the block-diagonal
 * update of the slides' backup frame "dropping precision correlations changes
 * the mean", App. A.3-A.5) for
 *
 *     L = sum(gy . y) + sum(gmuT . muT) + sum(gPT . PT),
 *
 * from the forward's inputs (it recomputes the states from checkpoints every
 * 8 tokens).  Per value row and key block, with h = P mu and the adjoints
 * (G_h, G_P) walked from the last token down: the readout adds w = P^-1 gy q
 * to G_h and -w mu^T to G_P; k gets (beta v) G_h + beta (G_P + G_P^T) k, the
 * write beta v gets G_h . k, beta's precision term k^T G_P k, the gate
 * <G_h, h_prev> + <G_P, P_prev> and tr G_P; both adjoints decay by alpha.
 *
 * Inputs (device pointers):
 *   q, k, v, beta, dt, A, I_prior, mu0, P0   as palimpsa_fwd_blockdiag
 *             (mu0 and P0 both given or both NULL: mu0 = 0, P0 = I_prior Id)
 *   gy        [B, T, H, dv]  gy_dtype   dL/dy
 *   gmuT      [B, H, dv, dk] float32    dL/dmuT, or NULL (zero)
 *   gPT       [B, H, dv, dk/block, block, block]  dL/dPT (every entry), or NULL (zero)
 * Outputs (float32, overwritten):
 *   gq, gk    [B, T, H, dk]     gv, gbeta [B, T, H, dv]     gdt [B, T, H]
 *   gA, gIp   [H]   summed over the batch; with the default start state gIp
 *             includes the start precision's share
 *   gmu0      [B, H, dv, dk]    dL/dmu0, or NULL
 *   gP0       [B, H, dv, dk/block, block, block]  the gradient for a symmetric
 *             P0 (written in full and symmetric: each off-diagonal pair holds
 *             half of the derivative by their shared value), or NULL
 *   flags     0, or PALIMPSA_CHECKPOINTS_SAVED: the workspace holds the
 *             checkpoints a palimpsa_fwd_blockdiag call with
 *             PALIMPSA_SAVE_CHECKPOINTS stored for the same inputs, and the
 *             checkpoint pass is skipped (the results are bitwise the same)
 *   workspace at least palimpsa_bwd_blockdiag_workspace_size(B, T, H, dk, dv,
 *             block) bytes, 16-byte aligned, caller-owned; contents on entry
 *             ignored unless PALIMPSA_CHECKPOINTS_SAVED
 *
 * block == 2 with dk in {32, 64, 128}, or block == 4 with dk in {64, 128}; dv a
 * multiple of 16 up to 1024 (else PALIMPSA_ERR_UNSUPPORTED).  A 4x4 block's
 * Cholesky factor serves both of its solves per token.  q, k, v, beta, gy, P0, gPT, gP0, gq, gk and the
 * workspace must be 16-byte aligned, the float32 arrays 4-byte aligned.
 * float32 arithmetic; results are deterministic (fixed reduction order).
 * T == 0 copies gmuT to gmu0 and the symmetric part of gPT to gP0.
 */
palimpsa_status palimpsa_bwd_blockdiag(const void *q, const void *k, const void *v, const void *beta,
                                       const void *dt, const float *A, const float *I_prior,
                                       const float *mu0, const float *P0,
                                       const void *gy, const float *gmuT, const float *gPT,
                                       float *gq, float *gk, float *gv, float *gbeta, float *gdt,
                                       float *gA, float *gIp, float *gmu0, float *gP0,
                                       int B, int T, int H, int dk, int dv, int block,
                                       int in_dtype, int gy_dtype, int flags,
                                       void *workspace, size_t workspace_bytes, void *stream);

/* Static, human-readable text for a status code (never NULL). */
const char *palimpsa_status_string(int status);

/* Library version as major * 10000 + minor * 100 + patch. */
int palimpsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PALIMPSA_H */
