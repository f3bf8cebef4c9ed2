/*
 * replayssm.h -- C ABI of the ReplaySSM decode-step library for AMD Instinct
 * MI355X (gfx950).
 *
 * Method: "NVIDIA ReplaySSM: hybrid model SSM decoding with a state buffer"
 * (devotd.net news article; section numbers below refer to its English
 * edition).  The SSM state of a sequence is kept as a checkpoint taken at the
 * start of an interval plus a buffer of the inputs of the tokens since then
 * (section 1).  Every token reads the checkpoint and replays the buffer to
 * form its output; the checkpoint is rewritten once per interval, when the
 * buffer is full.  Speculative verification produces outputs only and
 * rollback moves a buffer position (section 3).  An optional precision split
 * keeps a stochastically rounded update checkpoint and a separate 4-bit
 * output copy (section 4).
 *
 * The recurrence being replayed (per head h, group g = h / (H/G)):
 *     a_t = exp(dt_t * A_h)
 *     S_t = a_t * S_{t-1} + dt_t * x_t (outer) B_t       S: P x N
 *     y_t = S_t . C_t + D_h * x_t
 * and its replayed form after k buffered tokens j = 1..k since checkpoint S0:
 *     y_k = Lambda_k (S0 . C_k) + sum_j w_kj (B_j . C_k) x_j + D_h x_k
 *     S_k = Lambda_k S0 + sum_j w_kj x_j (outer) B_j
 * with l_i = A_h dt_i, Lambda_k = exp(sum_{i<=k} l_i) and
 * w_kj = dt_j exp(sum_{j<i<=k} l_i).
 *
 * Conventions for every call
 *  - Pointers named in rssm_state and the data arguments are DEVICE pointers
 *    unless stated otherwise; the rssm_desc / rssm_state structs themselves
 *    are host memory read during the call only.
 *  - All tensors are dense, row-major (last dimension innermost),
 *    little-endian.  The caller owns and allocates all memory; the library
 *    never allocates, frees or synchronises (except
 *    replayssm_check_device_errors) and never throws.
 *  - Every call is asynchronous on `stream`.  Calls that touch the same
 *    rssm_state must be issued on one stream (or otherwise ordered); calls on
 *    different states may run concurrently.
 *  - Return value: RSSM_OK, or a negative rssm_status.  Argument errors are
 *    detected on the host before anything is launched.  A failed launch
 *    returns RSSM_E_HIP.  The message of the last error of the calling thread
 *    is available from replayssm_last_error().
 *  - Device-side range errors (a position count out of range, n_keep > T, a
 *    row mapped to a slot outside 0..S-1) are clamped or skipped and
 *    recorded in a sticky flag read by
 *    replayssm_check_device_errors().  Two rows of one call mapped to the
 *    same slot race (results undefined); the position-publishing kernels
 *    flag it in the same word when they see it (more arrivals or marks on
 *    the slot than one row brings, or its position changed during the
 *    call).
 *
 * Shapes (B = batch, H = n_heads, P = head_dim, N = d_state, G = n_groups,
 * L = interval, Tmax = max_draft, Lcap = L + Tmax - 1):
 *   x    [B, H, P]          B, C  [B, G, N]         dt [B, H]     (in_dtype)
 *   speculative calls add a token axis after B: x [B, T, H, P] etc.
 *   y    [B, H, P] or [B, T, H, P]   fp32
 *   A, D [H] fp32
 *   ckpt [B, H, P, N] (ckpt_dtype)
 *   xbuf [B, Lcap, H, P]   bbuf [B, Lcap, G, N]   dtbuf [B, Lcap, H]   (in_dtype)
 *   pos, intv [B] int32;  work [B + 1] int32 (all zero before first use)
 *   (B here is the slot count S = n_slots; call inputs and outputs have
 *   `batch` rows, one per entry of slot_idx)
 *   out_q [B, H, P, N/2] uint8 (two FP4 codes per byte, even element in the
 *   low nibble);  out_scale [B, H, P, N/32] uint8 (E4M3 scale per 32 elements)
 *
 * Supported: P = 64, N = 128; in_dtype F32 or BF16; H % G == 0;
 * 1 <= L, 1 <= Tmax <= 8; Lcap <= 64 for step / accept / flush on F32
 * checkpoints; Lcap <= 32 for verify, deferred commits and the
 * low-precision formats (RSSM_E_CAPACITY otherwise).
 *
 * State formats (rssm_desc ckpt_dtype / out_dtype / shared_lowp):
 *   F32  / NONE / 0 : fp32 checkpoint (outputs and updates).
 *   BF16 or FP8_E4M3 / FP4_E2M1 / 0 : precision split (section 4): outputs
 *       read the FP4 copy; a commit forms the new state in fp32 from the
 *       update checkpoint and the buffer, stores it stochastically rounded
 *       into the update checkpoint and re-quantises the FP4 copy from the same
 *       fp32 values, so the copy's rounding never reaches later updates.
 *   NONE / FP4_E2M1 / 1 : the FP4 copy is the only state (ablation).
 *   BF16 or FP8_E4M3 / NONE / 0 : one rounded checkpoint for both.
 * Rounding: bf16 / E4M3 (OCP "FN", unscaled, saturating at 448) by
 * stochastic rounding -- up to the upper neighbour iff r16 / 2^16 <
 * (|v| - lo) / (hi - lo), r16 the 16-bit half (e mod 8) of Philox4x32-10
 * with key = seed and counter = (e / 8, interval, layer_id, 0), e the flat
 * element index in [B,H,P,N] and interval the index of the interval the
 * written state starts (intv[b] at load_checkpoint, intv[b] + 1 at a
 * commit).  FP4: E2M1 codes with one E4M3 scale RNE(amax / 6) per 32
 * consecutive elements of a row, codes RNE(|v| / scale) saturating at 6.
 * B*H*P*N must be < 2^32 for the low-precision formats.
 */
#ifndef REPLAYSSM_H_
#define REPLAYSSM_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rssm_status {
    RSSM_OK = 0,
    RSSM_E_ARG = -1,          /* null pointer, bad size, inconsistent descriptor */
    RSSM_E_UNSUPPORTED = -2,  /* shape / dtype combination not built */
    RSSM_E_CAPACITY = -3,     /* T > max_draft or Lcap too large */
    RSSM_E_HIP = -4,          /* a HIP runtime call failed */
    RSSM_E_DEVICE = -5        /* device-side range error recorded (sticky) */
} rssm_status;

typedef enum rssm_dtype {
    RSSM_F32 = 0,
    RSSM_BF16 = 1,
    RSSM_FP8_E4M3 = 2,        /* OCP FP8 E4M3 ("FN": no inf, max 448) */
    RSSM_FP4_E2M1 = 3,        /* OCP MX FP4 E2M1 with an E4M3 scale per 32 */
    RSSM_NONE = 4
} rssm_dtype;

/* Layer descriptor (host struct). */
typedef struct rssm_desc {
    int32_t batch;        /* rows of a call (one sequence each); without a slot map, row b is slot b */
    int32_t n_heads;      /* H */
    int32_t head_dim;     /* P */
    int32_t d_state;      /* N */
    int32_t n_groups;     /* G: B/C groups; heads h use group h / (H/G) */
    int32_t interval;     /* L: tokens per checkpoint interval (article: 16) */
    int32_t max_draft;    /* Tmax: largest T of a speculative round (1 if unused) */
    int32_t in_dtype;     /* rssm_dtype of x, B, C, dt and the buffers: F32 | BF16 */
    int32_t ckpt_dtype;   /* checkpoint: F32, or BF16 / FP8_E4M3 (stochastically rounded); NONE when shared_lowp */
    int32_t out_dtype;    /* NONE: outputs read ckpt; FP4_E2M1: separate output copy (needs a BF16/FP8 ckpt) */
    int32_t shared_lowp;  /* 1: the FP4 output copy is the only state (ablation; ckpt_dtype NONE) */
    int32_t layer_id;     /* stochastic-rounding stream: layer index */
    uint64_t seed;        /* stochastic-rounding stream: key */
    int32_t deferred_commit; /* 1: replayssm_accept_deferred may be used on this layer (F32 checkpoint,
                                max_draft >= 2, L + Tmax <= 32); verify then also runs the fold pass */
    int32_t n_slots;      /* state slots S held by the rssm_state buffers; 0 means S = batch.  A call
                             covers `batch` rows, mapped to slots by rssm_state.slot_idx */
} rssm_desc;

/* int32 words of rssm_state.commit_list for S state slots. */
#define RSSM_COMMIT_LIST_WORDS(S) (32 + 4 * (S))

/* Device buffers of one layer (host struct of device pointers). */
typedef struct rssm_state {
    void *ckpt;           /* [B,H,P,N] ckpt_dtype (2, 1 or 4 bytes per element); NULL when shared_lowp */
    void *out_q;          /* [B,H,P,N/2] u8 when out_dtype == FP4_E2M1, else NULL */
    void *out_scale;      /* [B,H,P,N/32] u8 (E4M3) when out_dtype == FP4_E2M1 */
    void *xbuf;           /* [B,Lcap,H,P] in_dtype */
    void *bbuf;           /* [B,Lcap,G,N] in_dtype */
    void *dtbuf;          /* [B,Lcap,H]   in_dtype */
    int32_t *pos;         /* [B] valid buffer entries since the checkpoint: 0..L-1 at rest,
                             up to Lcap after replayssm_accept_deferred */
    int32_t *intv;        /* [B] checkpoints written so far (the rounding stream's interval index) */
    int32_t *work;        /* [B+1] library scratch: per-slot arrival counters / marks + sticky error word; zero-initialise once */
    const float *A;       /* [H] decay rate, A < 0 */
    const float *D;       /* [H] skip weight */
    float *debug_prequant;/* optional [B,H,P,N] fp32: commit values before rounding (split path tests); NULL */
    const int32_t *slot_idx; /* [batch] device: state slot of each call row, -1 = padding row (nothing
                                read or written for it); NULL = row b uses slot b.  Slots of one call
                                must be distinct (a duplicate is flagged when detected, see above).
                                Rows mapped outside 0..S-1 are skipped and flagged */
    int32_t *commit_list; /* [RSSM_COMMIT_LIST_WORDS(S)] int32, zero-initialise once and leave to the
                             library afterwards: the slots whose interval a low-precision step,
                             accept or flush closes, committed by the call's second launch
                             (needed by replayssm_step, replayssm_accept and replayssm_commit
                             with BF16 / FP8 / shared-FP4 states, RSSM_E_ARG when NULL there;
                             unused, may be NULL, otherwise).  Calls on one state must not
                             overlap */
} rssm_state;

/*
 * Standard decode step (article sections 1-2): one token per slot.
 * For each slot with k = pos[b] buffered tokens: y = replayed output of the
 * (k+1)-th token of the interval.  If k + 1 < L the token's x, B, dt are
 * appended at buffer entry k and pos becomes k + 1.  If k + 1 == L the
 * checkpoint is rewritten in the same pass that reads it (S_L from the
 * replayed form above), pos becomes 0 and intv is incremented.
 * A slot with k >= L (left by replayssm_accept_deferred) is handled the
 * same way: the output replays all k + 1 tokens and the pass commits them
 * (pos = 0, intv + 1).
 * x [B,H,P], B, C [B,G,N], dt [B,H] (in_dtype); y [B,H,P] fp32.
 */
int replayssm_step(const rssm_desc *desc, const rssm_state *st, const void *x,
                   const void *B, const void *C, const void *dt, float *y,
                   hipStream_t stream);

/*
 * replayssm_step without the caller's arrival counters, for callers that
 * cannot allocate device memory at any point (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * kernels and results as replayssm_step (bit-identical outputs and state),
 * but the per-slot arrival counters and the low-precision states' commit
 * lists live in library scratch: a device array of 65536 counters and two
 * 65536-slot lists (1.25 MB) per GPU, set up on the first call on that device
 * and held until the process ends.  Of st->work only the sticky error word
 * work[n_slots] is used (read it with replayssm_check_device_errors as
 * usual); st->commit_list is not used.  Calls nothing that allocates.
 * Every call on one GPU shares that GPU's counters: calls that overlap on
 * one GPU (different streams, different layers) race and must be ordered by
 * the caller.  Returns RSSM_E_CAPACITY when the state holds more than 65536
 * slots, RSSM_E_HIP if the scratch cannot be set up.
 */
int replayssm_step_noalloc(const rssm_desc *desc, const rssm_state *st, const void *x,
                           const void *B, const void *C, const void *dt, float *y, hipStream_t stream);

/*
 * Speculative verification (article section 3): T draft positions per slot
 * are appended at buffer entries pos .. pos+T-1 and the outputs of all T
 * positions are produced from the checkpoint and the buffer; no state is
 * written and pos is unchanged.  Requires 1 <= T <= max_draft.
 * F32 checkpoints only: a slot with pos >= L (left by
 * replayssm_accept_deferred) has its accepted entries folded into the
 * checkpoint in the same pass that reads it (a commit: pos = 0, intv + 1),
 * and its drafts are appended at entries 0 .. T-1 of the next interval.
 * The outputs are bit-identical to those after an eager accept.
 * x [B,T,H,P], B, C [B,T,G,N], dt [B,T,H] (in_dtype); y [B,T,H,P] fp32.
 */
int replayssm_verify(const rssm_desc *desc, const rssm_state *st, int32_t T,
                     const void *x, const void *B, const void *C, const void *dt,
                     float *y, hipStream_t stream);

/*
 * Accept / rollback (article section 3): pos[b] += n_keep[b], so only the
 * first n_keep[b] verified positions stay valid; rejected entries are
 * simply overwritten later.  Slots whose count reaches L are committed (all
 * their buffered tokens folded into the checkpoint, pos = 0, intv + 1).
 * n_keep [B] int32 device, 0 <= n_keep <= T (larger values are clamped and
 * flagged).
 */
int replayssm_accept(const rssm_desc *desc, const rssm_state *st,
                     const int32_t *n_keep, int32_t T, hipStream_t stream);

/*
 * Deferred accept (article section 3, with the commit deferred): pos[b] +=
 * n_keep[b] and nothing else; the checkpoint is not touched.  A slot whose
 * count reaches L (up to Lcap = L + Tmax - 1 entries) is folded by the next
 * replayssm_step, replayssm_verify or replayssm_commit on it, inside the pass
 * that reads the checkpoint anyway, which saves one checkpoint read and
 * write per interval against replayssm_accept.  Like replayssm_accept it
 * follows a verify (pos <= L-1 on entry; flagged otherwise).  Requires
 * desc->deferred_commit = 1 (RSSM_E_ARG otherwise), which in turn requires
 * an F32 checkpoint and max_draft >= 2 (else RSSM_E_UNSUPPORTED) and
 * L + Tmax <= 32 (else RSSM_E_CAPACITY: a step on a slot left at Lcap
 * entries replays Lcap + 1).  Outputs and checkpoints of a verify after a
 * deferred accept are bit-identical to those after replayssm_accept.
 */
int replayssm_accept_deferred(const rssm_desc *desc, const rssm_state *st,
                              const int32_t *n_keep, int32_t T, hipStream_t stream);

/*
 * Flush: commit every slot with pos > 0 (checkpoint <- state after its
 * buffered tokens, pos = 0, intv + 1), including slots holding up to Lcap
 * entries after a deferred accept.  Slots with pos == 0 are untouched.
 */
int replayssm_commit(const rssm_desc *desc, const rssm_state *st, hipStream_t stream);

/*
 * Prefill (the state a slot decodes from summarizes its prompt; article
 * section 1): the Tp prompt tokens of every slot are run through the
 * recurrence starting from the checkpoint (from_zero = 0; the buffer must be
 * empty, pos == 0, flagged otherwise) or from a zero state (from_zero = 1).
 * The state after the prompt becomes the checkpoint (pos = 0, intv + 1).
 * When y is not NULL the outputs of all prompt tokens are written.  Each
 * head's state stays on chip for the whole prompt, which is processed in
 * 16-token chunks; with an F32 checkpoint, results are bit-identical to
 * decoding the prompt token by token with L = 16 and flushing at the end.
 * With a low-precision state (article section 4) the prompt runs in fp32 on
 * chip from the decoded update source (update checkpoint, or the FP4 copy of
 * the shared mode) and the final state is written once, like a commit: the
 * update checkpoint by stochastic rounding with stream index intv + 1, the
 * FP4 copy quantised from the same fp32 values (debug_prequant receives
 * them when set); the prompt outputs come from the fp32 recurrence.
 * x [B,Tp,H,P], B, C [B,Tp,G,N], dt [B,Tp,H] (in_dtype); y [B,Tp,H,P] fp32
 * or NULL (then C may be NULL).
 */
int replayssm_prefill(const rssm_desc *desc, const rssm_state *st, int32_t Tp,
                      int32_t from_zero, const void *x, const void *B,
                      const void *C, const void *dt, float *y, hipStream_t stream);

/*
 * Load a checkpoint from an fp32 state src [B,H,P,N] (device): writes ckpt
 * (and the output copy when configured), rounding with stream index intv[b]
 * for the split formats, and sets pos = 0.  For F32 checkpoints it is a copy.
 */
int replayssm_load_checkpoint(const rssm_desc *desc, const rssm_state *st,
                              const float *src, hipStream_t stream);

/*
 * Conventional decode step, the in-run baseline (article section 1: every
 * token reads and writes the whole state): state [B,H,P,N] fp32 is updated
 * in place, y [B,H,P] fp32.
 */
int replayssm_recurrent_step(const rssm_desc *desc, float *state, const void *x,
                             const void *B, const void *C, const void *dt,
                             const float *A, const float *D, float *y,
                             hipStream_t stream);

/*
 * Conventional speculative verification, the in-run baseline (article
 * section 3: a state copy is kept for every draft token).  pool
 * [B, Tmax+1, H, P, N] fp32 holds each slot's states; sel [B] int32 names the
 * current one.  The T per-token states are written to pool slots
 * (sel + 1 + t) mod (Tmax + 1), t = 0..T-1; y [B,T,H,P] fp32.
 */
int replayssm_recurrent_verify(const rssm_desc *desc, float *pool, const int32_t *sel,
                               int32_t T, const void *x, const void *B, const void *C,
                               const void *dt, const float *A, const float *D,
                               float *y, hipStream_t stream);

/* Baseline accept: sel[b] <- (sel[b] + n_keep[b]) mod (Tmax + 1) when
 * n_keep[b] > 0 (the kept state is the n_keep-th copy; 0 keeps the old one). */
int replayssm_recurrent_accept(const rssm_desc *desc, int32_t *sel,
                               const int32_t *n_keep, int32_t T, hipStream_t stream);

/* Buffer capacity Lcap = L + Tmax - 1 in entries (0 for an invalid desc). */
size_t replayssm_buffer_capacity(const rssm_desc *desc);

/* Validate a descriptor without launching anything: RSSM_OK or an error. */
int replayssm_check_desc(const rssm_desc *desc);

/* Static text for a status code. */
const char *replayssm_status_string(int status);

/* Message of the calling thread's last error ("" if none). */
const char *replayssm_last_error(void);

/* Synchronise `stream`, read and clear the sticky device error word of st
 * (work[n_slots]; n_slots = the state's slot count S): RSSM_OK,
 * RSSM_E_DEVICE (with the recorded condition in last_error) or RSSM_E_HIP. */
int replayssm_check_device_errors(const rssm_state *st, int32_t n_slots, hipStream_t stream);

/*
 * Self-check of the device conversions the low-precision commit relies on
 * (a diagnostic for the hardware, not a compute call).  For every fp32 bit
 * pattern p with begin <= p < end (end <= 2^32), NaNs skipped, it counts
 *   counts[0]: patterns where gfx950's f32 -> E2M1 conversion at unit scale
 *              differs from the exact round-to-nearest-even FP4 encoding
 *              (saturating at 6, sign kept) the quantiser defines; the commit
 *              takes FP4 codes from that conversion bracketed from both sides
 *              of |v| / scale (precision split, article section 4);
 *   counts[1]: patterns with |v| <= 0x7F7F0000 where bf16 stochastic rounding
 *              by integer addition differs from the selecting form (a draw
 *              hashed from the pattern);
 *   counts[2]: (pattern, draw) pairs, NaNs included, where the E4M3
 *              stochastic rounding the kernels use (carry form in the normal
 *              range, exact floor split below it) differs from the grid-split
 *              form (two draws per pattern: the hashed one and its
 *              complement).
 * counts: device array of 3 unsigned 64-bit counters, zeroed by the caller;
 * the kernel adds to them.  Asynchronous on stream; RSSM_E_ARG for a NULL
 * counts or begin > end or end > 2^32.  All counts are 0 on a conforming
 * device.
 */
int replayssm_check_conversions(uint64_t begin, uint64_t end, unsigned long long *counts, hipStream_t stream);

/*
 * Diagnostic: stream `bytes` (a multiple of 16) through HBM with the same
 * 16-byte non-temporal accesses as the state-streaming kernels, so callers
 * can time the practical ceiling next to the kernels' achieved bandwidth.
 * mode 0 = read src with 8 independent loads in flight per thread (dst
 * receives grid*256 floats of partial sums and must hold that many);
 * mode 1 = copy src -> dst (both `bytes` long), same depth; mode 2 = read
 * src as 32 KB blocks, one per wave, 16 loads in flight per lane (the step
 * kernel's shape; `bytes` a multiple of 32768; dst as for mode 0).  grid
 * workgroups of 256 threads in a grid-stride loop.  Asynchronous on stream;
 * RSSM_E_ARG for a bad mode, size or grid.
 */
int replayssm_hbm_probe(int32_t mode, const void *src, void *dst, size_t bytes, int32_t grid,
                        hipStream_t stream);

/* Library version string. */
const char *replayssm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* REPLAYSSM_H_ */
