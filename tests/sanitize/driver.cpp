// driver.cpp -- the host code of libsmcsd.so (argument validation, launch plans, workspace
// layouts of every entry point) and the CPU oracle, run under AddressSanitizer and
// UndefinedBehaviorSanitizer without a GPU. The kernels' launchers are stubs (stubs.cpp) that
// count calls and fail, so a valid call ends with SMCSD_ERR_DEVICE after passing validation.
// (smcsd_round_noalloc lives with its device buffer in a HIP source and is not built here.)
// Exit status 0 when every check passes; a sanitizer finding aborts the process.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "smcsd.h"

extern int g_stub_launches;

extern "C" {
double orc_row_logsumexp(const void*, int, int64_t, double);
double orc_row_tv(const void*, const void*, int, int64_t, double);
int32_t orc_row_gumbel_argmax(const void*, int, const float*, int64_t, float, double*);
int32_t orc_resample_request(int32_t, const double*, const double*, double, int32_t, double,
                             double*, double*, int32_t*, double*, double*);
int32_t orc_remap_request(int32_t, int32_t, const int32_t*, const int32_t*, int32_t*, int32_t*,
                          int32_t);
int32_t orc_round(int32_t, int32_t, int32_t, int64_t, int64_t, int32_t, const void*, const void*,
                  const int32_t*, const float*, const float*, const float*, int32_t, float,
                  const float*, double*, double*, double*, double*, int32_t*, int32_t*, int32_t*,
                  int32_t*, double*, int32_t, int32_t, const int32_t*, int32_t*, int32_t*, double*,
                  double*, const float*);
void orc_sd_verify(int32_t, int32_t, int32_t, int64_t, int64_t, int32_t, const void*, const void*,
                   const int32_t*, const float*, const float*, const float*, const float*,
                   int32_t*, int32_t*, double*, double*, int32_t*, double*);
void orc_gumbel_topk(int64_t, int64_t, int64_t, int32_t, const void*, const float*, const float*,
                     int32_t, int32_t*, double*, double*);
int32_t orc_bonus_resampled(int32_t, int32_t, int32_t, int64_t, int64_t, int32_t, const void*,
                            const float*, const int32_t*, const float*, int32_t*, double*);
int32_t orc_pages_advance(int32_t, int32_t, int32_t, int32_t, const int32_t*, const int32_t*,
                          int32_t*, int32_t, int32_t*, int32_t*, int32_t*, uint8_t*, int64_t,
                          int32_t, int32_t);
}

static int g_fail = 0;
#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++g_fail;                                                            \
        }                                                                        \
    } while (0)

// Fake, aligned, non-null device pointers: validation must reject or accept a call without
// touching them.
static void* fake(uintptr_t i) { return reinterpret_cast<void*>(0x10000000u + 0x100000u * i); }

static smcsd_round_args round_args(int32_t R, int32_t N, int32_t K, int32_t V) {
    smcsd_round_args a;
    std::memset(&a, 0, sizeof a);
    a.R = R;
    a.N = N;
    a.K = K;
    a.V = V;
    a.ld = (V + 7) / 8 * 8;
    a.dtype = SMCSD_BF16;
    a.mode = SMCSD_RESAMPLE_ALWAYS;
    a.ess_frac = 0.5f;
    a.target_logits = fake(1);
    a.draft_logits = fake(2);
    a.draft_tokens = static_cast<const int32_t*>(fake(3));
    a.temperature = static_cast<const float*>(fake(4));
    a.gumbel = static_cast<const float*>(fake(5));
    a.uniform = static_cast<const float*>(fake(6));
    a.log_weights = static_cast<float*>(fake(7));
    a.log_w_incr = static_cast<float*>(fake(8));
    a.log_norm = static_cast<float*>(fake(9));
    a.ess = static_cast<float*>(fake(10));
    a.resampled = static_cast<int32_t*>(fake(11));
    a.ancestors = static_cast<int32_t*>(fake(12));
    a.bonus = static_cast<int32_t*>(fake(13));
    a.tv = static_cast<float*>(fake(14));
    a.workspace = fake(0x100);
    a.workspace_bytes = size_t(1) << 40;
    return a;
}

static void abi_checks() {
    // workspace sizes over a grid of sizes, including the extremes of every argument
    const int32_t Rs[] = {0, 1, 64, 4096, INT32_MAX};
    const int32_t Ns[] = {0, 1, 32, SMCSD_MAX_N, SMCSD_MAX_N + 1, INT32_MAX};
    const int32_t Ks[] = {0, 1, 8, SMCSD_MAX_K, SMCSD_MAX_K + 1};
    const int32_t Vs[] = {0, 1, 7, 128256, 1048576, 1048577, INT32_MAX};
    for (int32_t R : Rs)
        for (int32_t N : Ns)
            for (int32_t K : Ks)
                for (int32_t V : Vs)
                    for (int dt = -1; dt <= 2; ++dt)
                        for (int tv = 0; tv < 2; ++tv) {
                            const size_t b = smcsd_workspace_size(R, N, K, V, dt, tv);
                            if (N < 1 || N > SMCSD_MAX_N || K < 1 || K > SMCSD_MAX_K || V < 1 ||
                                R < 0 || dt < 0 || dt > 1)
                                CHECK(b == 0);
                            (void)smcsd_verify_workspace_size(R, N, K, V, dt);
                            (void)smcsd_bonus_workspace_size(R, N, V, dt);
                            (void)smcsd_topk_workspace_size(R, V, dt, K);
                            (void)smcsd_pages_workspace_size(R, N, K, V);
                        }
    CHECK(smcsd_workspace_size(64, 32, 8, 128256, SMCSD_BF16, 1) > 0);
    CHECK(smcsd_workspace_size(64, 32, 8, 128256, SMCSD_BF16, 1) <= SMCSD_NOALLOC_SCRATCH_BYTES);

    // round: invalid arguments come back before any launch, valid ones reach the first launch
    struct Case {
        void (*edit)(smcsd_round_args&);
        smcsd_status want;
    };
    const Case cases[] = {
        {[](smcsd_round_args& a) { a.N = 0; }, SMCSD_ERR_ARG},
        {[](smcsd_round_args& a) { a.K = 0; }, SMCSD_ERR_ARG},
        {[](smcsd_round_args& a) { a.V = 0; }, SMCSD_ERR_ARG},
        {[](smcsd_round_args& a) { a.R = -1; }, SMCSD_ERR_ARG},
        {[](smcsd_round_args& a) { a.ld = a.V - 1; }, SMCSD_ERR_ARG},
        {[](smcsd_round_args& a) { a.ld = a.V + 4; }, SMCSD_ERR_ARG},
        {[](smcsd_round_args& a) { a.dtype = 2; }, SMCSD_ERR_ARG},
        {[](smcsd_round_args& a) { a.mode = 3; }, SMCSD_ERR_ARG},
        {[](smcsd_round_args& a) { a.reserved0 = 1; }, SMCSD_ERR_ARG},
        {[](smcsd_round_args& a) { a.N = SMCSD_MAX_N + 1; }, SMCSD_ERR_UNSUPPORTED},
        {[](smcsd_round_args& a) { a.K = SMCSD_MAX_K + 1; }, SMCSD_ERR_UNSUPPORTED},
        {[](smcsd_round_args& a) { a.target_logits = nullptr; }, SMCSD_ERR_ARG},
        {[](smcsd_round_args& a) { a.gumbel = reinterpret_cast<const float*>(0x10000008); }, SMCSD_ERR_ARG},
        {[](smcsd_round_args& a) { a.workspace = nullptr; }, SMCSD_ERR_WORKSPACE},
        {[](smcsd_round_args& a) { a.workspace_bytes = 100; }, SMCSD_ERR_WORKSPACE},
        {[](smcsd_round_args& a) { a.mode = SMCSD_RESAMPLE_ESS; a.ess_frac = 0.0f; }, SMCSD_ERR_ARG},
        {[](smcsd_round_args& a) { a.V = 1048584; a.ld = 1048584; }, SMCSD_ERR_UNSUPPORTED},
        {[](smcsd_round_args& a) { a.R = INT32_MAX; a.N = SMCSD_MAX_N; a.K = SMCSD_MAX_K; }, SMCSD_ERR_UNSUPPORTED},
        {[](smcsd_round_args& a) {
             a.page_table_in = static_cast<const int32_t*>(fake(20));
             a.page_table_out = static_cast<int32_t*>(fake(20));
             a.P = 4;
             a.num_pages = 10;
         },
         SMCSD_ERR_ARG},
        {[](smcsd_round_args&) {}, SMCSD_ERR_DEVICE},
        {[](smcsd_round_args& a) { a.tv = nullptr; a.gumbel = nullptr; a.bonus = nullptr; }, SMCSD_ERR_DEVICE},
        {[](smcsd_round_args& a) {
             a.page_table_in = static_cast<const int32_t*>(fake(20));
             a.page_table_out = static_cast<int32_t*>(fake(40));
             a.refcount = static_cast<int32_t*>(fake(60));
             a.P = 256;
             a.num_pages = 1 << 20;
         },
         SMCSD_ERR_DEVICE},
    };
    for (const Case& c : cases) {
        smcsd_round_args a = round_args(64, 32, 8, 128256);
        c.edit(a);
        const int before = g_stub_launches;
        const smcsd_status st = smcsd_round(&a, nullptr);
        CHECK(st == c.want);
        CHECK((g_stub_launches > before) == (c.want == SMCSD_ERR_DEVICE));
    }
    smcsd_round_args empty = round_args(0, 8, 4, 100);
    empty.target_logits = nullptr;
    CHECK(smcsd_round(&empty, nullptr) == SMCSD_OK);
    CHECK(smcsd_round(nullptr, nullptr) == SMCSD_ERR_ARG);

    // the other entry points
    const float* f = static_cast<const float*>(fake(1));
    float* fo = static_cast<float*>(fake(2));
    int32_t* io = static_cast<int32_t*>(fake(3));
    CHECK(smcsd_resample(1, 0, f, fo, f, 0, 0.5f, fo, fo, io, io, nullptr) == SMCSD_ERR_ARG);
    CHECK(smcsd_resample(2, SMCSD_MAX_N, f, fo, f, 1, 0.5f, fo, fo, io, io, nullptr) == SMCSD_ERR_DEVICE);
    CHECK(smcsd_remap_pages(1, 4, 4, io, io, io, io, 10, nullptr, nullptr) == SMCSD_ERR_ARG);
    CHECK(smcsd_remap_pages(3, 16, 2048, io, static_cast<int32_t*>(fake(30)), static_cast<int32_t*>(fake(60)),
                            io, 1 << 20, nullptr, nullptr) == SMCSD_ERR_DEVICE);
    CHECK(smcsd_remap_pages(INT32_MAX, SMCSD_MAX_N, INT32_MAX, io, static_cast<int32_t*>(fake(30)),
                            static_cast<int32_t*>(fake(90)), io, 10, nullptr, nullptr) != SMCSD_OK);
    CHECK(smcsd_gumbel_topk(4, 1000, 1000, SMCSD_BF16, fake(1), f, f, 0, io, fo, fake(0x100), 1 << 20,
                            nullptr) == SMCSD_ERR_ARG);
    CHECK(smcsd_gumbel_topk(4, 1000, 1000, SMCSD_BF16, fake(1), f, f, SMCSD_MAX_TOPK + 1, io, fo,
                            fake(0x100), 1 << 20, nullptr) != SMCSD_OK);
    CHECK(smcsd_gumbel_topk(2048, 128256, 128256, SMCSD_BF16, fake(1), f, f, 8, io, fo, fake(0x100),
                            size_t(1) << 30, nullptr) == SMCSD_ERR_DEVICE);
    CHECK(smcsd_bonus_resampled(2, 8, 4, 1000, 1000, SMCSD_BF16, fake(1), f, io, f, io, nullptr,
                                fake(0x100), size_t(1) << 30, nullptr, nullptr) == SMCSD_ERR_DEVICE);
    CHECK(smcsd_bonus_resampled(2, 0, 4, 1000, 1000, SMCSD_BF16, fake(1), f, io, f, io, nullptr,
                                fake(0x100), size_t(1) << 30, nullptr, nullptr) == SMCSD_ERR_ARG);
    // page table, refcount, free list, its count: 1 MiB each at most, disjoint
    int32_t* ptab = static_cast<int32_t*>(fake(3));
    int32_t* rcnt = static_cast<int32_t*>(fake(80));
    int32_t* fids = static_cast<int32_t*>(fake(90));
    int32_t* nf = static_cast<int32_t*>(fake(100));
    CHECK(smcsd_pages_advance(8, 16, 2048, 16, io, io, ptab, 1 << 18, rcnt, fids, nf, fake(70), 32768,
                              64, int64_t(1) << 33, 0, fake(0x100), size_t(1) << 30, nullptr, nullptr,
                              nullptr) == SMCSD_ERR_DEVICE);
    CHECK(smcsd_pages_advance(8, 16, 2048, 0, io, io, ptab, 1 << 18, rcnt, fids, nf, fake(70), 32768,
                              64, int64_t(1) << 33, 0, fake(0x100), size_t(1) << 30, nullptr, nullptr,
                              nullptr) == SMCSD_ERR_ARG);
    CHECK(smcsd_pages_advance(8, 16, 2048, 16, io, io, ptab, 1 << 18, ptab, fids, nf, fake(70), 32768,
                              64, int64_t(1) << 33, 0, fake(0x100), size_t(1) << 30, nullptr, nullptr,
                              nullptr) == SMCSD_ERR_ARG);   // refcount aliases the page table
    smcsd_verify_args v;
    std::memset(&v, 0, sizeof v);
    v.R = 2;
    v.N = 8;
    v.K = 4;
    v.V = 1000;
    v.ld = 1000;
    v.dtype = SMCSD_BF16;
    v.target_logits = fake(1);
    v.draft_logits = fake(2);
    v.draft_tokens = io;
    v.temperature = f;
    v.gumbel = f;
    v.accept_uniform = f;
    v.residual_uniform = f;
    v.n_accepted = io;
    v.next_token = io;
    v.workspace = fake(0x100);
    v.workspace_bytes = size_t(1) << 30;
    CHECK(smcsd_sd_verify(&v, nullptr) == SMCSD_ERR_DEVICE);
    v.reserved0 = 1;
    CHECK(smcsd_sd_verify(&v, nullptr) == SMCSD_ERR_ARG);
    for (int32_t s = -1; s <= 6; ++s) CHECK(smcsd_status_string(s) != nullptr);
    CHECK(std::strcmp(smcsd_status_string(99), "unknown status") == 0);
}

// bf16 bit patterns of values drawn from a normal distribution
static std::vector<uint16_t> bf16_rows(std::mt19937& g, size_t n, float sd) {
    std::normal_distribution<float> d(0.0f, sd);
    std::vector<uint16_t> out(n);
    for (size_t i = 0; i < n; ++i) {
        const float x = d(g);
        uint32_t b;
        std::memcpy(&b, &x, 4);
        out[i] = static_cast<uint16_t>(b >> 16);
    }
    return out;
}

static void oracle_checks() {
    std::mt19937 g(7);
    std::uniform_real_distribution<float> uni(0.0f, 1.0f);
    for (int trial = 0; trial < 6; ++trial) {
        const int32_t R = 1 + trial % 3, N = 1 + 7 * trial, K = 1 + trial % 4;
        const int64_t V = 5 + 97 * trial, ld = (V + 7) / 8 * 8;
        const int32_t P = 3 + trial;
        std::vector<uint16_t> tgt = bf16_rows(g, size_t(R) * N * (K + 1) * ld, 2.0f);
        std::vector<uint16_t> dft = bf16_rows(g, size_t(R) * N * K * ld, 2.0f);
        std::vector<int32_t> tok(size_t(R) * N * K);
        for (auto& t : tok) t = static_cast<int32_t>(g() % V);
        std::vector<float> T(R, 0.8f), gum(size_t(R) * N * ld), u(R), lwin(size_t(R) * N, -std::log((float)N));
        for (auto& x : gum) x = -std::log(-std::log(std::fmin(std::fmax(uni(g), 1e-7f), 1.0f - 1e-7f)));
        for (auto& x : u) x = uni(g) * 0.999f;
        std::vector<float> lpot(size_t(R) * N);
        for (auto& x : lpot) x = uni(g) - 0.5f;
        if (N > 1) lpot[0] = -INFINITY;    // a removed particle (one must stay)
        std::vector<int32_t> pt(size_t(R) * N * P), pt_out(pt.size());
        const int32_t pages = R * N * P + 5;
        for (size_t i = 0; i < pt.size(); ++i) pt[i] = (i % 5 == 4) ? -1 : static_cast<int32_t>(i);
        std::vector<int32_t> rc(pages, 0);
        for (int32_t p : pt)
            if (p >= 0) ++rc[p];
        std::vector<double> lw(size_t(R) * N), lwo(lw.size()), lnorm(R), ess(R), tv(size_t(R) * N * K),
            ag(lw.size()), bg(lw.size());
        std::vector<int32_t> rs(R), anc(lw.size()), bonus(lw.size()), ot(size_t(R) * N * (K + 1));
        for (int mode = 0; mode < 3; ++mode) {
            std::vector<int32_t> rc2 = rc;
            const int32_t st = orc_round(R, N, K, V, ld, 1, tgt.data(), dft.data(), tok.data(), T.data(),
                                         gum.data(), u.data(), mode, 0.5f, lwin.data(), lw.data(),
                                         lwo.data(), lnorm.data(), ess.data(), rs.data(), anc.data(),
                                         bonus.data(), ot.data(), tv.data(), P, pages, pt.data(),
                                         pt_out.data(), rc2.data(), ag.data(), bg.data(),
                                         mode == 1 ? lpot.data() : nullptr);
            CHECK(st == 0);
            for (size_t i = 0; i < anc.size(); ++i) CHECK(anc[i] >= 0 && anc[i] < N);
            for (double x : tv) CHECK(x >= 0.0 && x <= 1.0 + 1e-12);
        }
        // sd verification, top-k, bonus after resampling
        std::vector<float> au(size_t(R) * N * K), bu(size_t(R) * N);
        for (auto& x : au) x = uni(g);
        for (auto& x : bu) x = uni(g);
        std::vector<int32_t> nacc(size_t(R) * N), next(nacc.size()), nb(2 * nacc.size());
        std::vector<double> accg(nacc.size()), res(2 * nacc.size()), bgap(nacc.size());
        orc_sd_verify(R, N, K, V, ld, 1, tgt.data(), dft.data(), tok.data(), T.data(), gum.data(),
                      au.data(), bu.data(), nacc.data(), next.data(), accg.data(), res.data(), nb.data(),
                      bgap.data());
        for (size_t i = 0; i < nacc.size(); ++i) CHECK(nacc[i] >= 0 && nacc[i] <= K && next[i] >= 0 && next[i] < V);
        const int32_t k = static_cast<int32_t>(std::min<int64_t>(V, 9));
        const int64_t rows = int64_t(R) * N;
        std::vector<float> Tr(rows, 1.1f);
        std::vector<int32_t> ttok(rows * k);
        std::vector<double> tkey(rows * k), tgap(rows * k);
        orc_gumbel_topk(rows, V, ld, 1, dft.data(), Tr.data(), gum.data(), k, ttok.data(), tkey.data(),
                        tgap.data());
        for (int64_t r = 0; r < rows; ++r)
            for (int32_t j = 1; j < k; ++j) CHECK(tkey[r * k + j] <= tkey[r * k + j - 1]);
        std::vector<int32_t> anc2(rows), b2(rows);
        for (int64_t i = 0; i < rows; ++i) anc2[i] = static_cast<int32_t>(g() % N);
        anc2[0] = N;                                        // out of range: flagged
        CHECK(orc_bonus_resampled(R, N, K, V, ld, 1, tgt.data(), T.data(), anc2.data(), gum.data(),
                                  b2.data(), bg.data()) == -1);
        CHECK(b2[0] == -1);
    }
    // resampling alone at every N up to the maximum, and the remap's range checks
    for (int32_t N : {1, 2, 63, 64, 65, 333, SMCSD_MAX_N}) {
        std::vector<double> lw(N), prev(N, -std::log((double)N)), lwn(N), gap(N);
        for (auto& x : lw) x = 3.0 * (uni(g) - 0.5);
        std::vector<int32_t> anc(N);
        double logZ, ess;
        orc_resample_request(N, lw.data(), prev.data(), 0.37, 0, 0.5, &logZ, &ess, anc.data(), lwn.data(),
                             gap.data());
        for (int32_t j = 1; j < N; ++j) CHECK(anc[j] >= anc[j - 1]);
        std::vector<int32_t> pt(size_t(N) * 3), out(pt.size()), rc(size_t(N) * 3 + 1, 0);
        for (size_t i = 0; i < pt.size(); ++i) {
            pt[i] = static_cast<int32_t>(i);
            rc[i] = 1;
        }
        CHECK(orc_remap_request(N, 3, anc.data(), pt.data(), out.data(), rc.data(), (int32_t)rc.size()) == 0);
        anc[0] = N;
        CHECK(orc_remap_request(N, 3, anc.data(), pt.data(), out.data(), rc.data(), (int32_t)rc.size()) == -1);
    }
    // page lifecycle: copy-on-write, appends, an exhausted free list, token-major copies
    for (int token_rows = 0; token_rows < 2; ++token_rows) {
        const int32_t R = 2, N = 5, P = 6, ps = 4, pages = 40, kvc = 3;
        const int64_t page_bytes = 32;
        std::vector<int32_t> pt(size_t(R) * N * P, -1), rc(pages, -1), fl(pages);
        int32_t nfree = 0;
        for (int32_t r = 0; r < R; ++r)
            for (int32_t j = 0; j < N; ++j) {
                pt[(size_t(r) * N + j) * P + 0] = r * 10;        // shared prompt page
                pt[(size_t(r) * N + j) * P + 1] = r * 10 + 1;    // shared, partly filled tail
            }
        for (int32_t p = 0; p < pages; ++p) {
            int32_t c = 0;
            for (int32_t e : pt) c += e == p;
            rc[p] = c > 0 ? c : -1;
            if (c == 0) fl[nfree++] = p;
        }
        std::vector<uint8_t> kv(size_t(kvc) * pages * page_bytes);
        for (size_t i = 0; i < kv.size(); ++i) kv[i] = static_cast<uint8_t>(i * 7);
        const int32_t lb[2] = {6, 5}, la[2] = {11, 9};
        const int32_t st = orc_pages_advance(R, N, P, ps, lb, la, pt.data(), pages, rc.data(), fl.data(),
                                             &nfree, kv.data(), page_bytes, kvc, token_rows);
        CHECK(st == 0 || st == -3);
        CHECK(nfree >= 0 && nfree <= pages);
        int32_t small_free = 1;
        std::vector<int32_t> pt2 = pt, rc2 = rc, fl2 = fl;
        const int32_t st2 = orc_pages_advance(R, N, P, ps, la, la, pt2.data(), pages, rc2.data(), fl2.data(),
                                              &small_free, kv.data(), page_bytes, kvc, token_rows);
        CHECK(st2 == 0 || st2 == -3);
    }
    // single rows: the closed forms the pins rely on
    const float z[3] = {4.0f, 1.0f, 2.5f};
    const float g0[3] = {0.0f, 0.0f, 0.0f};
    double gap = 0.0;
    CHECK(orc_row_gumbel_argmax(z, 0, g0, 3, 0.5f, &gap) == 0);
    CHECK(std::fabs(gap - 3.0) < 1e-12);
    CHECK(std::fabs(orc_row_logsumexp(z, 0, 1, 1.0) - 4.0) < 1e-12);
    CHECK(orc_row_tv(z, z, 0, 3, 0.7) == 0.0);
}

int main() {
    abi_checks();
    oracle_checks();
    if (g_fail) {
        std::fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    std::printf("sanitized host checks passed (%d stub launches)\n", g_stub_launches);
    return 0;
}
