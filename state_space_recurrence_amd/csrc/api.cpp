// api.cpp -- extern "C" entry points of libreplayssm: argument validation on
// the host, then asynchronous kernel launches.  See include/replayssm.h for
// the contract of every call.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "replayssm.h"
#include "kernels.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return RSSM_OK;
    return fail(RSSM_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxLcap = 64;       // step / accept / flush on F32 checkpoints
constexpr int kMaxLcapVerify = 32; // verify, deferred commits and the low-precision formats
constexpr int kMaxDraft = 8;

int lcap_of(const rssm_desc *d) { return d->interval + d->max_draft - 1; }

// State slots held by the buffers (rssm_desc.n_slots, 0 = batch).
int nslots_of(const rssm_desc *d) { return d->n_slots > 0 ? d->n_slots : d->batch; }

int heads_per_wg(const rssm_desc *d) {
    const int hpg = d->n_heads / d->n_groups;
    return hpg % 4 == 0 ? 4 : (hpg % 2 == 0 ? 2 : 1);
}

// Low-precision mode of a descriptor (rssm::SplitMode), or -1 for the fp32
// checkpoint path.
int split_mode(const rssm_desc *d) {
    if (d->shared_lowp) return rssm::kSharedFP4;
    if (d->ckpt_dtype == RSSM_BF16) return d->out_dtype == RSSM_FP4_E2M1 ? rssm::kSplitBF16 : rssm::kLowBF16;
    if (d->ckpt_dtype == RSSM_FP8_E4M3) return d->out_dtype == RSSM_FP4_E2M1 ? rssm::kSplitE4M3 : rssm::kLowE4M3;
    return -1;
}

// Deferred accepts (declared by desc->deferred_commit) can leave up to Lcap
// entries in a slot; a step on such a slot replays and commits one more.
bool deferred_ok(const rssm_desc *d) { return d->deferred_commit == 1; }

int check_desc(const rssm_desc *d) {
    if (!d) return fail(RSSM_E_ARG, "desc is NULL");
    if (d->batch < 0) return fail(RSSM_E_ARG, "batch %d < 0", d->batch);
    if (d->n_slots < 0) return fail(RSSM_E_ARG, "n_slots %d < 0", d->n_slots);
    if (d->n_heads <= 0 || d->n_groups <= 0)
        return fail(RSSM_E_ARG, "n_heads %d / n_groups %d must be positive", d->n_heads, d->n_groups);
    if (d->n_heads % d->n_groups != 0)
        return fail(RSSM_E_ARG, "n_heads %d not a multiple of n_groups %d", d->n_heads, d->n_groups);
    if (d->head_dim != 64 || d->d_state != 128)
        return fail(RSSM_E_UNSUPPORTED, "head_dim %d x d_state %d: only 64 x 128 is built",
                    d->head_dim, d->d_state);
    if (d->interval < 1) return fail(RSSM_E_ARG, "interval %d < 1", d->interval);
    if (d->max_draft < 1 || d->max_draft > kMaxDraft)
        return fail(RSSM_E_CAPACITY, "max_draft %d outside 1..%d", d->max_draft, kMaxDraft);
    if (lcap_of(d) > kMaxLcap)
        return fail(RSSM_E_CAPACITY, "interval + max_draft - 1 = %d exceeds %d", lcap_of(d), kMaxLcap);
    if (d->in_dtype != RSSM_F32 && d->in_dtype != RSSM_BF16)
        return fail(RSSM_E_UNSUPPORTED, "in_dtype %d: only F32 and BF16 inputs", d->in_dtype);
    if (d->shared_lowp != 0 && d->shared_lowp != 1)
        return fail(RSSM_E_ARG, "shared_lowp must be 0 or 1");
    if (d->out_dtype != RSSM_NONE && d->out_dtype != RSSM_FP4_E2M1)
        return fail(RSSM_E_UNSUPPORTED, "out_dtype %d: only NONE or FP4_E2M1", d->out_dtype);
    if (d->shared_lowp) {
        if (d->out_dtype != RSSM_FP4_E2M1 || d->ckpt_dtype != RSSM_NONE)
            return fail(RSSM_E_ARG, "shared_lowp needs out_dtype FP4_E2M1 and ckpt_dtype NONE "
                                    "(the FP4 copy is the only state)");
    } else {
        if (d->ckpt_dtype != RSSM_F32 && d->ckpt_dtype != RSSM_BF16 && d->ckpt_dtype != RSSM_FP8_E4M3)
            return fail(RSSM_E_UNSUPPORTED, "ckpt_dtype %d: F32, BF16 or FP8_E4M3", d->ckpt_dtype);
        if (d->ckpt_dtype == RSSM_F32 && d->out_dtype != RSSM_NONE)
            return fail(RSSM_E_UNSUPPORTED, "an FP4 output copy goes with a BF16 / FP8 update checkpoint");
    }
    if (d->deferred_commit != 0 && d->deferred_commit != 1)
        return fail(RSSM_E_ARG, "deferred_commit must be 0 or 1");
    if (d->deferred_commit) {
        if (split_mode(d) >= 0)
            return fail(RSSM_E_UNSUPPORTED, "deferred_commit: F32 checkpoints only");
        if (d->max_draft < 2)
            return fail(RSSM_E_UNSUPPORTED, "deferred_commit: needs max_draft >= 2 (speculative rounds)");
        if (lcap_of(d) + 1 > kMaxLcapVerify)
            return fail(RSSM_E_CAPACITY, "deferred_commit: interval + max_draft = %d exceeds %d",
                        d->interval + d->max_draft, kMaxLcapVerify);
    }
    if ((int64_t)d->batch * d->n_heads > (int64_t)1 << 24 || (int64_t)nslots_of(d) * d->n_heads > (int64_t)1 << 24)
        return fail(RSSM_E_ARG, "batch * n_heads or n_slots * n_heads too large");
    if (split_mode(d) >= 0 && lcap_of(d) > kMaxLcapVerify)
        return fail(RSSM_E_CAPACITY, "low-precision state: interval + max_draft - 1 = %d exceeds %d",
                    lcap_of(d), kMaxLcapVerify);
    if (split_mode(d) >= 0 && (int64_t)nslots_of(d) * d->n_heads * d->head_dim * d->d_state > 0xFFFFFFFFll)
        return fail(RSSM_E_ARG, "low-precision state: B*H*P*N must fit the 32-bit element index of the "
                                "rounding stream");
    return RSSM_OK;
}

int check_state(const rssm_desc *d, const rssm_state *s) {
    if (!s) return fail(RSSM_E_ARG, "state is NULL");
    if (d->batch == 0) return RSSM_OK;
    if (!d->shared_lowp && !s->ckpt) return fail(RSSM_E_ARG, "state->ckpt is NULL");
    if (d->out_dtype == RSSM_FP4_E2M1 && (!s->out_q || !s->out_scale))
        return fail(RSSM_E_ARG, "state->out_q / out_scale are NULL with an FP4 output copy");
    if (!s->xbuf || !s->bbuf || !s->dtbuf) return fail(RSSM_E_ARG, "state buffers are NULL");
    if (!s->pos || !s->intv || !s->work) return fail(RSSM_E_ARG, "state pos/intv/work is NULL");
    if (!s->A || !s->D) return fail(RSSM_E_ARG, "state A/D is NULL");
    if (!s->slot_idx && d->batch > nslots_of(d))
        return fail(RSSM_E_ARG, "batch %d exceeds n_slots %d without a slot map", d->batch, nslots_of(d));
    return RSSM_OK;
}

rssm::ReplayParams replay_params(const rssm_desc *d, const rssm_state *s) {
    rssm::ReplayParams p{};
    p.ckpt = static_cast<float *>(s->ckpt);
    p.xbuf = s->xbuf;
    p.bbuf = s->bbuf;
    p.dtbuf = s->dtbuf;
    p.pos = s->pos;
    p.intv = s->intv;
    p.work = s->work;
    p.err = s->work + nslots_of(d);
    p.clist = s->commit_list;
    p.A = s->A;
    p.D = s->D;
    p.batch = d->batch;
    p.slot_idx = s->slot_idx;
    p.nslots = nslots_of(d);
    p.H = d->n_heads;
    p.G = d->n_groups;
    p.L = d->interval;
    p.Lcap = lcap_of(d);
    p.kmax = deferred_ok(d) ? p.Lcap : d->interval - 1;
    p.T = 1;
    p.hpw = heads_per_wg(d);
    p.wg_per_slot = d->n_heads / p.hpw;
    p.u = s->ckpt;
    p.oq = static_cast<uint8_t *>(s->out_q);
    p.os = static_cast<uint8_t *>(s->out_scale);
    p.dbg = s->debug_prequant;
    p.seed = d->seed;
    p.layer = d->layer_id;
    return p;
}

#define RSSM_TRY(expr)              \
    do {                            \
        int rc_ = (expr);           \
        if (rc_ != RSSM_OK) return rc_; \
    } while (0)

// Low-precision step: outputs and appends, then the commit pass over the
// slots whose interval that step closed.
int split_step(const rssm::ReplayParams &p, bool bf, int mode, hipStream_t stream) {
    RSSM_TRY(hip_status(rssm::launch_split_step(p, bf, mode, stream), "split step launch"));
    return hip_status(rssm::launch_split_commit_list(p, bf, mode, stream), "split commit launch");
}

}  // namespace

extern "C" {

int replayssm_check_desc(const rssm_desc *desc) {
    g_last_error[0] = 0;
    return check_desc(desc);
}

size_t replayssm_buffer_capacity(const rssm_desc *desc) {
    if (check_desc(desc) != RSSM_OK) return 0;
    return (size_t)lcap_of(desc);
}

int replayssm_step(const rssm_desc *desc, const rssm_state *st, const void *x, const void *B,
                   const void *C, const void *dt, float *y, hipStream_t stream) {
    RSSM_TRY(check_desc(desc));
    RSSM_TRY(check_state(desc, st));
    if (desc->batch == 0) return RSSM_OK;
    if (!x || !B || !C || !dt || !y) return fail(RSSM_E_ARG, "step: an input/output pointer is NULL");
    rssm::ReplayParams p = replay_params(desc, st);
    p.x = x;
    p.Bm = B;
    p.Cm = C;
    p.dt = dt;
    p.y = y;
    const bool bf = desc->in_dtype == RSSM_BF16;
    const int mode = split_mode(desc);
    if (mode >= 0) {
        if (!st->commit_list) return fail(RSSM_E_ARG, "step: a low-precision state needs state->commit_list");
        return split_step(p, bf, mode, stream);
    }
    return hip_status(rssm::launch_replay_step(p, bf, stream), "replay step launch");
}

int replayssm_step_noalloc(const rssm_desc *desc, const rssm_state *st, const void *x, const void *B,
                           const void *C, const void *dt, float *y, hipStream_t stream) {
    RSSM_TRY(check_desc(desc));
    if (nslots_of(desc) > rssm::kNoAllocMaxSlots)
        return fail(RSSM_E_CAPACITY, "step_noalloc: %d state slots exceed the library scratch (%d slots)",
                    nslots_of(desc), rssm::kNoAllocMaxSlots);
    RSSM_TRY(check_state(desc, st));
    if (desc->batch == 0) return RSSM_OK;
    if (!x || !B || !C || !dt || !y) return fail(RSSM_E_ARG, "step_noalloc: an input/output pointer is NULL");
    rssm::ReplayParams p = replay_params(desc, st);
    RSSM_TRY(hip_status(rssm::noalloc_work(&p.work, &p.clist, stream), "step_noalloc: library scratch"));
    p.x = x;
    p.Bm = B;
    p.Cm = C;
    p.dt = dt;
    p.y = y;
    const bool bf = desc->in_dtype == RSSM_BF16;
    const int mode = split_mode(desc);
    if (mode >= 0) return split_step(p, bf, mode, stream);
    return hip_status(rssm::launch_replay_step(p, bf, stream), "replay step launch");
}

int replayssm_verify(const rssm_desc *desc, const rssm_state *st, int32_t T, const void *x,
                     const void *B, const void *C, const void *dt, float *y, hipStream_t stream) {
    RSSM_TRY(check_desc(desc));
    if (T < 1 || T > desc->max_draft)
        return fail(RSSM_E_CAPACITY, "verify: T = %d outside 1..max_draft (%d)", T, desc->max_draft);
    if (lcap_of(desc) > kMaxLcapVerify)
        return fail(RSSM_E_CAPACITY, "verify: interval + max_draft - 1 = %d exceeds %d", lcap_of(desc),
                    kMaxLcapVerify);
    RSSM_TRY(check_state(desc, st));
    if (desc->batch == 0) return RSSM_OK;
    if (!x || !B || !C || !dt || !y) return fail(RSSM_E_ARG, "verify: an input/output pointer is NULL");
    rssm::ReplayParams p = replay_params(desc, st);
    p.x = x;
    p.Bm = B;
    p.Cm = C;
    p.dt = dt;
    p.y = y;
    p.T = T;
    const bool bf = desc->in_dtype == RSSM_BF16;
    const int mode = split_mode(desc);
    if (mode >= 0) return hip_status(rssm::launch_split_verify(p, bf, mode, stream), "split verify launch");
    return hip_status(rssm::launch_replay_verify(p, bf, stream), "replay verify launch");
}

int replayssm_accept(const rssm_desc *desc, const rssm_state *st, const int32_t *n_keep, int32_t T,
                     hipStream_t stream) {
    RSSM_TRY(check_desc(desc));
    if (T < 1 || T > desc->max_draft)
        return fail(RSSM_E_CAPACITY, "accept: T = %d outside 1..max_draft (%d)", T, desc->max_draft);
    RSSM_TRY(check_state(desc, st));
    if (desc->batch == 0) return RSSM_OK;
    if (!n_keep) return fail(RSSM_E_ARG, "accept: n_keep is NULL");
    rssm::ReplayParams p = replay_params(desc, st);
    p.n_keep = n_keep;
    p.T = T;
    const bool bf = desc->in_dtype == RSSM_BF16;
    const int mode = split_mode(desc);
    if (mode >= 0) {
        if (!st->commit_list) return fail(RSSM_E_ARG, "accept: a low-precision state needs state->commit_list");
        return hip_status(rssm::launch_split_accept(p, bf, mode, true, stream), "split accept launch");
    }
    return hip_status(rssm::launch_replay_commit(p, bf, true, stream), "accept launch");
}

int replayssm_accept_deferred(const rssm_desc *desc, const rssm_state *st, const int32_t *n_keep, int32_t T,
                              hipStream_t stream) {
    RSSM_TRY(check_desc(desc));
    if (T < 1 || T > desc->max_draft)
        return fail(RSSM_E_CAPACITY, "accept_deferred: T = %d outside 1..max_draft (%d)", T, desc->max_draft);
    if (!deferred_ok(desc))
        return fail(RSSM_E_ARG, "accept_deferred: the descriptor does not declare deferred_commit");
    RSSM_TRY(check_state(desc, st));
    if (desc->batch == 0) return RSSM_OK;
    if (!n_keep) return fail(RSSM_E_ARG, "accept_deferred: n_keep is NULL");
    rssm::ReplayParams p = replay_params(desc, st);
    p.n_keep = n_keep;
    p.T = T;
    return hip_status(rssm::launch_defer_accept(p, stream), "deferred accept launch");
}

int replayssm_commit(const rssm_desc *desc, const rssm_state *st, hipStream_t stream) {
    RSSM_TRY(check_desc(desc));
    RSSM_TRY(check_state(desc, st));
    if (desc->batch == 0) return RSSM_OK;
    rssm::ReplayParams p = replay_params(desc, st);
    const bool bf = desc->in_dtype == RSSM_BF16;
    const int mode = split_mode(desc);
    if (mode >= 0) {
        if (!st->commit_list) return fail(RSSM_E_ARG, "commit: a low-precision state needs state->commit_list");
        return hip_status(rssm::launch_split_accept(p, bf, mode, false, stream), "split commit launch");
    }
    return hip_status(rssm::launch_replay_commit(p, bf, false, stream), "commit launch");
}

int replayssm_prefill(const rssm_desc *desc, const rssm_state *st, int32_t Tp, int32_t from_zero, const void *x,
                      const void *B, const void *C, const void *dt, float *y, hipStream_t stream) {
    RSSM_TRY(check_desc(desc));
    if (Tp < 0) return fail(RSSM_E_ARG, "prefill: Tp = %d < 0", Tp);
    if (from_zero != 0 && from_zero != 1) return fail(RSSM_E_ARG, "prefill: from_zero must be 0 or 1");
    if ((int64_t)desc->batch * Tp * desc->n_heads > (int64_t)1 << 31)
        return fail(RSSM_E_ARG, "prefill: batch * Tp * n_heads too large");
    RSSM_TRY(check_state(desc, st));
    if (desc->batch == 0 || Tp == 0) return RSSM_OK;
    if (!x || !B || !dt) return fail(RSSM_E_ARG, "prefill: x / B / dt is NULL");
    if (y && !C) return fail(RSSM_E_ARG, "prefill: outputs need C");
    rssm::ReplayParams p = replay_params(desc, st);
    p.x = x;
    p.Bm = B;
    p.Cm = C;
    p.dt = dt;
    p.y = y;
    p.T = Tp;
    p.from_zero = from_zero;
    return hip_status(rssm::launch_prefill(p, desc->in_dtype == RSSM_BF16, y != nullptr, split_mode(desc), stream),
                      "prefill launch");
}

int replayssm_load_checkpoint(const rssm_desc *desc, const rssm_state *st, const float *src,
                              hipStream_t stream) {
    RSSM_TRY(check_desc(desc));
    RSSM_TRY(check_state(desc, st));
    if (desc->batch == 0) return RSSM_OK;
    if (!src) return fail(RSSM_E_ARG, "load_checkpoint: src is NULL");
    const int mode = split_mode(desc);
    if (mode >= 0) {
        rssm::ReplayParams p = replay_params(desc, st);
        p.src = src;
        p.dbg = nullptr;
        RSSM_TRY(hip_status(rssm::launch_split_load(p, mode, stream), "load_checkpoint quantise"));
        return hip_status(rssm::launch_zero_pos(p, stream), "load_checkpoint pos reset");
    }
    rssm::ReplayParams p = replay_params(desc, st);
    p.src = src;
    if (st->slot_idx) {
        RSSM_TRY(hip_status(rssm::launch_load_f32(p, stream), "load_checkpoint copy"));
    } else {
        const size_t bytes = (size_t)desc->batch * desc->n_heads * desc->head_dim * desc->d_state * sizeof(float);
        RSSM_TRY(hip_status(hipMemcpyAsync(st->ckpt, src, bytes, hipMemcpyDeviceToDevice, stream),
                            "load_checkpoint copy"));
    }
    return hip_status(rssm::launch_zero_pos(p, stream), "load_checkpoint pos reset");
}

int replayssm_recurrent_step(const rssm_desc *desc, float *state, const void *x, const void *B,
                             const void *C, const void *dt, const float *A, const float *D, float *y,
                             hipStream_t stream) {
    RSSM_TRY(check_desc(desc));
    if (desc->batch == 0) return RSSM_OK;
    if (!state || !x || !B || !C || !dt || !A || !D || !y)
        return fail(RSSM_E_ARG, "recurrent_step: a pointer is NULL");
    rssm::RecurrentParams p{};
    p.state = state;
    p.x = x;
    p.Bm = B;
    p.Cm = C;
    p.dt = dt;
    p.A = A;
    p.D = D;
    p.y = y;
    p.batch = desc->batch;
    p.H = desc->n_heads;
    p.G = desc->n_groups;
    p.T = 1;
    p.Tmax = desc->max_draft;
    p.hpw = heads_per_wg(desc);
    p.wg_per_slot = desc->n_heads / p.hpw;
    return hip_status(rssm::launch_recurrent(p, desc->in_dtype == RSSM_BF16, false, stream),
                      "recurrent step launch");
}

int replayssm_recurrent_verify(const rssm_desc *desc, float *pool, const int32_t *sel, int32_t T,
                               const void *x, const void *B, const void *C, const void *dt,
                               const float *A, const float *D, float *y, hipStream_t stream) {
    RSSM_TRY(check_desc(desc));
    if (T < 1 || T > desc->max_draft)
        return fail(RSSM_E_CAPACITY, "recurrent_verify: T = %d outside 1..max_draft (%d)", T, desc->max_draft);
    if (desc->batch == 0) return RSSM_OK;
    if (!pool || !sel || !x || !B || !C || !dt || !A || !D || !y)
        return fail(RSSM_E_ARG, "recurrent_verify: a pointer is NULL");
    rssm::RecurrentParams p{};
    p.state = pool;
    p.sel = sel;
    p.x = x;
    p.Bm = B;
    p.Cm = C;
    p.dt = dt;
    p.A = A;
    p.D = D;
    p.y = y;
    p.batch = desc->batch;
    p.H = desc->n_heads;
    p.G = desc->n_groups;
    p.T = T;
    p.Tmax = desc->max_draft;
    p.hpw = heads_per_wg(desc);
    p.wg_per_slot = desc->n_heads / p.hpw;
    return hip_status(rssm::launch_recurrent(p, desc->in_dtype == RSSM_BF16, true, stream),
                      "recurrent verify launch");
}

int replayssm_recurrent_accept(const rssm_desc *desc, int32_t *sel, const int32_t *n_keep, int32_t T,
                               hipStream_t stream) {
    RSSM_TRY(check_desc(desc));
    if (T < 1 || T > desc->max_draft)
        return fail(RSSM_E_CAPACITY, "recurrent_accept: T = %d outside 1..max_draft (%d)", T, desc->max_draft);
    if (desc->batch == 0) return RSSM_OK;
    if (!sel || !n_keep) return fail(RSSM_E_ARG, "recurrent_accept: a pointer is NULL");
    return hip_status(rssm::launch_recurrent_accept(sel, n_keep, desc->batch, T, desc->max_draft, stream),
                      "recurrent accept launch");
}

const char *replayssm_status_string(int status) {
    switch (status) {
        case RSSM_OK: return "ok";
        case RSSM_E_ARG: return "invalid argument";
        case RSSM_E_UNSUPPORTED: return "unsupported configuration";
        case RSSM_E_CAPACITY: return "capacity exceeded";
        case RSSM_E_HIP: return "HIP runtime error";
        case RSSM_E_DEVICE: return "device-side range error";
        default: return "unknown status";
    }
}

const char *replayssm_last_error(void) { return g_last_error; }

int replayssm_check_device_errors(const rssm_state *st, int32_t n_slots, hipStream_t stream) {
    if (!st || !st->work) return fail(RSSM_E_ARG, "check_device_errors: state/work is NULL");
    const int32_t batch = n_slots;
    if (batch < 0) return fail(RSSM_E_ARG, "check_device_errors: n_slots < 0");
    RSSM_TRY(hip_status(hipStreamSynchronize(stream), "check_device_errors sync"));
    int32_t word = 0;
    RSSM_TRY(hip_status(hipMemcpy(&word, st->work + batch, sizeof(word), hipMemcpyDeviceToHost),
                        "check_device_errors read"));
    if (word == 0) return RSSM_OK;
    const int32_t zero = 0;
    RSSM_TRY(hip_status(hipMemcpy(st->work + batch, &zero, sizeof(zero), hipMemcpyHostToDevice),
                        "check_device_errors clear"));
    return fail(RSSM_E_DEVICE,
                "device range error flags 0x%x (1: position out of range, 2: n_keep out of range, "
                "4: row mapped to a slot out of range, 8: two rows of one call on the same slot)",
                word);
}

int replayssm_hbm_probe(int32_t mode, const void *src, void *dst, size_t bytes, int32_t grid,
                        hipStream_t stream) {
    if (mode < 0 || mode > 2)
        return fail(RSSM_E_ARG, "hbm_probe: mode must be 0 (read), 1 (copy) or 2 (read, 32 KB per wave)");
    if (!src || !dst) return fail(RSSM_E_ARG, "hbm_probe: NULL buffer");
    if (bytes % 16 != 0 || bytes == 0) return fail(RSSM_E_ARG, "hbm_probe: bytes must be a positive multiple of 16");
    if (mode == 2 && bytes % 32768 != 0) return fail(RSSM_E_ARG, "hbm_probe: mode 2 needs a multiple of 32 KB");
    if (grid < 1 || grid > (1 << 20)) return fail(RSSM_E_ARG, "hbm_probe: grid outside 1..2^20");
    return hip_status(rssm::launch_probe(mode, static_cast<const float *>(src), static_cast<float *>(dst), bytes,
                                         grid, stream),
                      "hbm probe launch");
}

int replayssm_check_conversions(uint64_t begin, uint64_t end, unsigned long long *counts, hipStream_t stream) {
    if (!counts) return fail(RSSM_E_ARG, "check_conversions: NULL counts");
    if (end > (1ull << 32) || begin > end) return fail(RSSM_E_ARG, "check_conversions: need begin <= end <= 2^32");
    return hip_status(rssm::launch_conversion_check(begin, end, counts, stream), "conversion check launch");
}

const char *replayssm_version(void) { return "replayssm-gfx950 0.3"; }

}  // extern "C"
