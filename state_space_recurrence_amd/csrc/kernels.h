// kernels.h -- host-side launch interface of the ReplaySSM HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rssm {

// Arguments shared by the replay kernels (fp32 checkpoint path).
struct ReplayParams {
    float *ckpt;            // [B,H,P,N] fp32 checkpoint
    const void *x;          // [B,T,H,P] in dtype
    const void *Bm;         // [B,T,G,N]
    const void *Cm;         // [B,T,G,N]
    const void *dt;         // [B,T,H]
    float *y;               // [B,T,H,P] fp32
    void *xbuf;             // [B,Lcap,H,P]
    void *bbuf;             // [B,Lcap,G,N]
    void *dtbuf;            // [B,Lcap,H]
    int32_t *pos;           // [B]
    int32_t *intv;          // [B]
    int32_t *work;          // [nslots] per-slot arrival counters (zero between calls)
    int32_t *err;           // sticky device error word (work[nslots] of the caller's state)
    int32_t *clist;         // low-precision step: slots whose interval closed (see kListHead)
    const float *A;         // [H]
    const float *D;         // [H]
    const int32_t *n_keep;  // [B] (accept)
    int batch, H, G, L, Lcap, T;
    int kmax;               // largest pos a step / verify accepts: L-1, or Lcap with deferred accepts
    const int32_t *slot_idx;  // [batch] state slot of each call row, -1 = padding row; NULL = identity
    int nslots;             // state slots (ckpt / buffers / pos / intv / arrival counters)
    int from_zero;          // prefill: start from a zero state instead of the checkpoint
    int hpw;                // heads (waves) per workgroup
    int wg_per_slot;        // H / hpw
    // precision split (ignored by the fp32 kernels)
    void *u;                // update checkpoint [B,H,P,N]: bf16 (u16) or E4M3 (u8); NULL when shared
    uint8_t *oq;            // FP4 output copy codes [B,H,P,N/2]
    uint8_t *os;            // FP4 output copy scales [B,H,P,N/32] (E4M3)
    float *dbg;             // optional pre-rounding dump [B,H,P,N] fp32
    const float *src;       // load_checkpoint source [B,H,P,N] fp32
    uint64_t seed;
    int layer;
};

// Low-precision state modes of the precision split.
enum SplitMode {
    kSplitBF16 = 0,   // outputs read the FP4 copy; updates read/write a bf16 checkpoint (SR)
    kSplitE4M3 = 1,   // same with an E4M3 update checkpoint
    kSharedFP4 = 2,   // the FP4 copy is the only state (outputs and updates)
    kLowBF16 = 3,     // one bf16 checkpoint serves outputs and updates (no copy)
    kLowE4M3 = 4,     // one E4M3 checkpoint serves outputs and updates (no copy)
};

// Arguments of the conventional (recurrent) baseline kernels.
struct RecurrentParams {
    float *state;           // [B,H,P,N] (in place) or pool [B,Tmax+1,H,P,N]
    const int32_t *sel;     // [B] current pool slot (pool mode)
    const void *x, *Bm, *Cm, *dt;
    const float *A, *D;
    float *y;
    int batch, H, G, T, Tmax;
    int hpw, wg_per_slot;
};

// Launchers; in_bf16 selects bf16 inputs (else fp32).  Return hipError_t.
hipError_t launch_replay_step(const ReplayParams &p, bool in_bf16, hipStream_t s);
hipError_t launch_replay_verify(const ReplayParams &p, bool in_bf16, hipStream_t s);
hipError_t launch_replay_commit(const ReplayParams &p, bool in_bf16, bool accept, hipStream_t s);
hipError_t launch_zero_pos(const ReplayParams &p, hipStream_t s);
hipError_t launch_load_f32(const ReplayParams &p, hipStream_t s);   // ckpt[slot] <- src[row]
hipError_t launch_defer_accept(const ReplayParams &p, hipStream_t s);
// p.T = prompt length; mode -1 = fp32 checkpoint, else the SplitMode of a low-precision state
hipError_t launch_prefill(const ReplayParams &p, bool in_bf16, bool outputs, int mode, hipStream_t s);
hipError_t launch_split_step(const ReplayParams &p, bool in_bf16, int mode, hipStream_t s);
hipError_t launch_split_verify(const ReplayParams &p, bool in_bf16, int mode, hipStream_t s);
hipError_t launch_split_load(const ReplayParams &p, int mode, hipStream_t s);
hipError_t launch_recurrent(const RecurrentParams &p, bool in_bf16, bool pool, hipStream_t s);
hipError_t launch_conversion_check(uint64_t begin, uint64_t end, unsigned long long *counts, hipStream_t stream);
hipError_t launch_probe(int mode, const float *src, float *dst, size_t bytes, int grid, hipStream_t s);
hipError_t launch_recurrent_accept(int32_t *sel, const int32_t *n_keep, int batch, int T,
                                   int Tmax, hipStream_t s);

// Commit lists of the low-precision step (int32, kListHead + 4 x slots
// words): two lists used in turn, so that the commit pass never clears the
// count it reads.  [0], [1] entries in list 0 / 1; [kListFill] the list the
// next step fills; [kListLast] the list the last step filled; list e's
// entries (slot | entries << kListCountShift, new interval index) from
// kListHead + 2 e slots (a slot index fits 24 bits: the rounding draws'
// element index of a pool fits 32).  Zero at creation; afterwards the words
// between calls are the library's.  Accepts and flushes use the same lists.
constexpr int kListFill = 2;
constexpr int kListLast = 3;
constexpr int kListHead = 32;
constexpr int kListCountShift = 24;
constexpr int kListSlotMask = (1 << kListCountShift) - 1;
constexpr long list_words(long slots) { return kListHead + 4 * slots; }
hipError_t launch_split_commit_list(const ReplayParams &p, bool in_bf16, int mode, hipStream_t s);
// Accept (n_keep) or flush for the low-precision formats: positions and the
// commit list in one small launch, then the commit pass over the list.
hipError_t launch_split_accept(const ReplayParams &p, bool in_bf16, int mode, bool accept, hipStream_t s);

// Library scratch for callers that cannot allocate: per-slot arrival counters
// of up to kNoAllocMaxSlots slots and the commit lists of as many slots, one
// array per device.  *work / *clist receive the current device's copies (set
// up, and cleared on `s`, on its first use).
constexpr int kNoAllocMaxSlots = 1 << 16;
hipError_t noalloc_work(int32_t **work, int32_t **clist, hipStream_t s);

}  // namespace rssm
