// Host-side checks of the C ABI under AddressSanitizer / UndefinedBehavior-
// Sanitizer, without a GPU: every entry point is called with arguments its
// host validation must refuse (or with an empty batch), so no launch is ever
// reached.  The kernel launchers are replaced by stubs that abort, so a call
// that would have launched fails the run.  Built with g++ (host code only)
// from the library's api.cpp by tests/test_sanitizers.py.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kernels.h"
#include "replayssm.h"

namespace rssm {
#define RSSM_STUB(sig)                                                   \
    sig {                                                                \
        std::fprintf(stderr, "a kernel launch was reached: %s\n", #sig); \
        std::abort();                                                    \
    }
RSSM_STUB(hipError_t launch_replay_step(const ReplayParams &, bool, hipStream_t))
RSSM_STUB(hipError_t launch_replay_verify(const ReplayParams &, bool, hipStream_t))
RSSM_STUB(hipError_t launch_replay_commit(const ReplayParams &, bool, bool, hipStream_t))
RSSM_STUB(hipError_t launch_zero_pos(const ReplayParams &, hipStream_t))
RSSM_STUB(hipError_t launch_load_f32(const ReplayParams &, hipStream_t))
RSSM_STUB(hipError_t launch_defer_accept(const ReplayParams &, hipStream_t))
RSSM_STUB(hipError_t launch_prefill(const ReplayParams &, bool, bool, int, hipStream_t))
RSSM_STUB(hipError_t launch_split_step(const ReplayParams &, bool, int, hipStream_t))
RSSM_STUB(hipError_t launch_split_verify(const ReplayParams &, bool, int, hipStream_t))
RSSM_STUB(hipError_t launch_split_accept(const ReplayParams &, bool, int, bool, hipStream_t))
RSSM_STUB(hipError_t launch_split_load(const ReplayParams &, int, hipStream_t))
RSSM_STUB(hipError_t launch_recurrent(const RecurrentParams &, bool, bool, hipStream_t))
RSSM_STUB(hipError_t launch_probe(int, const float *, float *, size_t, int, hipStream_t))
RSSM_STUB(hipError_t launch_conversion_check(uint64_t, uint64_t, unsigned long long *, hipStream_t))
RSSM_STUB(hipError_t launch_recurrent_accept(int32_t *, const int32_t *, int, int, int, hipStream_t))
RSSM_STUB(hipError_t noalloc_work(int32_t **, int32_t **, hipStream_t))
RSSM_STUB(hipError_t launch_split_commit_list(const ReplayParams &, bool, int, hipStream_t))
}  // namespace rssm

static int g_checks = 0, g_fail = 0;

static void expect(const char *what, int rc, int want) {
    ++g_checks;
    const bool ok = want == RSSM_OK ? rc == RSSM_OK : (want == 1 ? rc != RSSM_OK : rc == want);
    if (!ok) {
        ++g_fail;
        std::fprintf(stderr, "FAIL %s: rc %d (want %d) last_error '%s'\n", what, rc, want,
                     replayssm_last_error());
    }
    // the message of a refusal is a terminated, non-empty string
    if (rc != RSSM_OK && std::strlen(replayssm_last_error()) == 0) {
        ++g_fail;
        std::fprintf(stderr, "FAIL %s: empty last_error\n", what);
    }
}

static rssm_desc good_desc() {
    rssm_desc d;
    std::memset(&d, 0, sizeof(d));
    d.batch = 4; d.n_heads = 8; d.head_dim = 64; d.d_state = 128; d.n_groups = 1;
    d.interval = 16; d.max_draft = 5; d.in_dtype = RSSM_BF16; d.ckpt_dtype = RSSM_F32;
    d.out_dtype = RSSM_NONE; d.seed = 7;
    return d;
}

int main() {
    alignas(16) static char mem[1 << 12];   // stands in for device buffers; never dereferenced
    void *p = mem;
    rssm_state st;
    std::memset(&st, 0, sizeof(st));
    st.ckpt = p; st.xbuf = p; st.bbuf = p; st.dtbuf = p;
    st.pos = (int32_t *)p; st.intv = (int32_t *)p; st.work = (int32_t *)p;
    st.A = (const float *)p; st.D = (const float *)p;
    rssm_state empty;
    std::memset(&empty, 0, sizeof(empty));
    const hipStream_t s = nullptr;
    float *y = (float *)p;

    // descriptors
    expect("good desc", replayssm_check_desc(nullptr), RSSM_E_ARG);
    rssm_desc d = good_desc();
    expect("good desc", replayssm_check_desc(&d), RSSM_OK);
    struct { const char *what; void (*edit)(rssm_desc &); int want; } bad[] = {
        {"head_dim", [](rssm_desc &d) { d.head_dim = 32; }, RSSM_E_UNSUPPORTED},
        {"d_state", [](rssm_desc &d) { d.d_state = 64; }, RSSM_E_UNSUPPORTED},
        {"groups", [](rssm_desc &d) { d.n_heads = 6; d.n_groups = 4; }, RSSM_E_ARG},
        {"no groups", [](rssm_desc &d) { d.n_groups = 0; }, RSSM_E_ARG},
        {"batch", [](rssm_desc &d) { d.batch = -1; }, RSSM_E_ARG},
        {"n_slots", [](rssm_desc &d) { d.n_slots = -3; }, RSSM_E_ARG},
        {"interval", [](rssm_desc &d) { d.interval = 0; }, RSSM_E_ARG},
        {"max_draft", [](rssm_desc &d) { d.max_draft = 0; }, RSSM_E_CAPACITY},
        {"max_draft big", [](rssm_desc &d) { d.max_draft = 9; }, RSSM_E_CAPACITY},
        {"lcap", [](rssm_desc &d) { d.interval = 64; d.max_draft = 2; }, RSSM_E_CAPACITY},
        {"in dtype", [](rssm_desc &d) { d.in_dtype = RSSM_FP8_E4M3; }, RSSM_E_UNSUPPORTED},
        {"out dtype", [](rssm_desc &d) { d.out_dtype = RSSM_BF16; }, RSSM_E_UNSUPPORTED},
        {"fp32 + copy", [](rssm_desc &d) { d.out_dtype = RSSM_FP4_E2M1; }, RSSM_E_UNSUPPORTED},
        {"shared flag", [](rssm_desc &d) { d.shared_lowp = 2; }, RSSM_E_ARG},
        {"shared needs fp4", [](rssm_desc &d) { d.shared_lowp = 1; }, RSSM_E_ARG},
        {"ckpt dtype", [](rssm_desc &d) { d.ckpt_dtype = 17; }, RSSM_E_UNSUPPORTED},
        {"deferred flag", [](rssm_desc &d) { d.deferred_commit = 3; }, RSSM_E_ARG},
        {"deferred lowp", [](rssm_desc &d) { d.deferred_commit = 1; d.ckpt_dtype = RSSM_BF16; }, RSSM_E_UNSUPPORTED},
        {"deferred T", [](rssm_desc &d) { d.deferred_commit = 1; d.max_draft = 1; }, RSSM_E_UNSUPPORTED},
        {"deferred cap", [](rssm_desc &d) { d.deferred_commit = 1; d.interval = 28; }, RSSM_E_CAPACITY},
        {"lowp cap", [](rssm_desc &d) { d.ckpt_dtype = RSSM_BF16; d.interval = 40; d.max_draft = 1; }, RSSM_E_CAPACITY},
        {"too big", [](rssm_desc &d) { d.batch = 1 << 22; }, RSSM_E_ARG},
        {"lowp index", [](rssm_desc &d) { d.ckpt_dtype = RSSM_BF16; d.batch = 8192; d.n_heads = 128; d.n_groups = 8; }, RSSM_E_ARG},
    };
    for (auto &b : bad) {
        rssm_desc e = good_desc();
        b.edit(e);
        expect(b.what, replayssm_check_desc(&e), b.want);
        expect(b.what, replayssm_step(&e, &st, p, p, p, p, y, s), b.want);
        expect(b.what, replayssm_commit(&e, &st, s), b.want);
        expect(b.what, (int)(replayssm_buffer_capacity(&e) == 0 ? b.want : RSSM_OK), b.want);
    }
    expect("capacity", (int)replayssm_buffer_capacity(&d) - 20, RSSM_OK);

    // states and pointers
    expect("step null state", replayssm_step(&d, nullptr, p, p, p, p, y, s), RSSM_E_ARG);
    expect("step empty state", replayssm_step(&d, &empty, p, p, p, p, y, s), RSSM_E_ARG);
    expect("step null x", replayssm_step(&d, &st, nullptr, p, p, p, y, s), RSSM_E_ARG);
    expect("step null y", replayssm_step(&d, &st, p, p, p, p, nullptr, s), RSSM_E_ARG);
    expect("noalloc null y", replayssm_step_noalloc(&d, &st, p, p, p, p, nullptr, s), RSSM_E_ARG);
    rssm_desc many = good_desc();
    many.batch = 70000;
    expect("noalloc capacity", replayssm_step_noalloc(&many, &st, p, p, p, p, y, s), RSSM_E_CAPACITY);
    rssm_desc nob = good_desc();
    nob.batch = 0;
    expect("step empty batch", replayssm_step(&nob, &st, nullptr, nullptr, nullptr, nullptr, nullptr, s), RSSM_OK);
    expect("verify empty batch", replayssm_verify(&nob, &st, 3, nullptr, nullptr, nullptr, nullptr, nullptr, s),
           RSSM_OK);
    expect("verify T 0", replayssm_verify(&d, &st, 0, p, p, p, p, y, s), RSSM_E_CAPACITY);
    expect("verify T big", replayssm_verify(&d, &st, 6, p, p, p, p, y, s), RSSM_E_CAPACITY);
    expect("verify null", replayssm_verify(&d, &st, 2, p, nullptr, p, p, y, s), RSSM_E_ARG);
    expect("accept null keep", replayssm_accept(&d, &st, nullptr, 2, s), RSSM_E_ARG);
    expect("accept T", replayssm_accept(&d, &st, (const int32_t *)p, 7, s), 1);
    expect("deferred undeclared", replayssm_accept_deferred(&d, &st, (const int32_t *)p, 2, s), 1);
    // a low-precision state without its commit lists is refused before any launch
    rssm_desc lp = good_desc();
    lp.ckpt_dtype = RSSM_BF16;
    lp.out_dtype = RSSM_FP4_E2M1;
    rssm_state lst = st;
    lst.out_q = p;
    lst.out_scale = p;
    lst.commit_list = nullptr;
    expect("lowp step lists", replayssm_step(&lp, &lst, p, p, p, p, y, s), RSSM_E_ARG);
    expect("lowp accept lists", replayssm_accept(&lp, &lst, (const int32_t *)p, 2, s), RSSM_E_ARG);
    expect("lowp commit lists", replayssm_commit(&lp, &lst, s), RSSM_E_ARG);
    expect("prefill Tp", replayssm_prefill(&d, &st, -1, 0, p, p, p, p, y, s), 1);
    expect("prefill null", replayssm_prefill(&d, &st, 5, 0, nullptr, p, p, p, y, s), RSSM_E_ARG);
    expect("load null", replayssm_load_checkpoint(&d, &st, nullptr, s), RSSM_E_ARG);
    expect("recurrent null", replayssm_recurrent_step(&d, nullptr, p, p, p, p, (const float *)p, (const float *)p,
                                                      y, s), RSSM_E_ARG);
    expect("recurrent verify", replayssm_recurrent_verify(&d, (float *)p, nullptr, 2, p, p, p, p,
                                                          (const float *)p, (const float *)p, y, s), RSSM_E_ARG);
    expect("recurrent accept", replayssm_recurrent_accept(&d, nullptr, (const int32_t *)p, 2, s), RSSM_E_ARG);
    expect("device errors null", replayssm_check_device_errors(nullptr, 4, s), RSSM_E_ARG);
    expect("probe mode", replayssm_hbm_probe(3, p, p, 1 << 20, 16, s), RSSM_E_ARG);
    expect("probe size", replayssm_hbm_probe(0, p, p, 15, 16, s), RSSM_E_ARG);
    expect("probe head size", replayssm_hbm_probe(2, p, p, 1 << 12, 16, s), RSSM_E_ARG);
    expect("probe grid", replayssm_hbm_probe(0, p, p, 1 << 12, 0, s), RSSM_E_ARG);
    for (int code = -6; code <= 1; ++code) {
        const char *m = replayssm_status_string(code);
        ++g_checks;
        if (!m || !*m) { ++g_fail; std::fprintf(stderr, "FAIL status string %d\n", code); }
    }
    ++g_checks;
    if (!replayssm_version() || !*replayssm_version()) ++g_fail;
    std::printf("%d host checks, %d failed\n", g_checks, g_fail);
    return g_fail ? 1 : 0;
}
