// abi_driver.cpp -- drives the C ABI's host-side validation (kda_api.cpp,
// linked in with launch_stubs.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer.
//
// Part 1 checks the status code of representative argument errors of every
// entry point (include/kda.h documents them).  Part 2 sweeps every integer
// argument of every entry point over extreme values (negative, zero, one,
// the 128 boundaries, KDA_MAX_HEADS + 1, INT32_MAX, huge token counts) and
// requires a valid status code: the size arithmetic of the validation must
// neither overflow a signed type nor read out of bounds for any input.
// Pointers are fake device addresses that validation never dereferences;
// calls that pass validation reach a stub launcher and return
// KDA_ERR_DEVICE.  Exit status 0 when every check passes.  Test
// infrastructure only.
#include <stdint.h>
#include <stdio.h>

#include <climits>
#include <functional>
#include <vector>

#include "kda.h"

namespace {

int failures = 0;

void expect(const char* what, int got, int want) {
    if (got != want) {
        fprintf(stderr, "FAIL: %s returned %d, expected %d\n", what, got, want);
        ++failures;
    }
}

void expect_valid(const char* what, int got) {
    if (got < KDA_OK || got > KDA_ERR_DEVICE) {
        fprintf(stderr, "FAIL: %s returned out-of-range status %d\n", what, got);
        ++failures;
    }
}

// fake, 16-byte aligned, far-apart device addresses
void* P(int i, uintptr_t off = 0) {
    return reinterpret_cast<void*>((uintptr_t(1) << 40) + uintptr_t(i) * (uintptr_t(1) << 36) + off);
}
float* F(int i, uintptr_t off = 0) { return static_cast<float*>(P(i, off)); }
const int32_t* I(int i, uintptr_t off = 0) { return static_cast<const int32_t*>(P(i, off)); }

struct ChunkA {
    void *q = P(0), *k = P(1), *v = P(2), *g = P(3), *b = P(4);
    float* h0 = F(5);
    const int32_t* cu = I(6);
    int32_t N = 1;
    int64_t T = 64;
    int32_t H = 2, Dk = 128, Dv = 128;
    int dt = KDA_BF16;
    void* o = P(7);
    float* hT = F(8);
    int32_t chunk = 0, split = 0;
    int call() const {
        return kda_chunk_fwd_ex(q, k, v, g, b, h0, cu, N, T, H, Dk, Dv, (kda_dtype)dt, o, hT,
                                nullptr, 0, chunk, split, nullptr);
    }
};

struct DecodeA {
    void *q = P(0), *k = P(1), *v = P(2), *g = P(3), *b = P(4);
    float* S = F(5);
    int32_t B = 4, H = 2, Dk = 128, Dv = 128;
    int dt = KDA_BF16;
    void* o = P(6);
    int call() const {
        return kda_decode_step(q, k, v, g, b, S, B, H, Dk, Dv, (kda_dtype)dt, o, nullptr);
    }
};

struct MultiA {
    void *q = P(0), *k = P(1), *v = P(2), *g = P(3), *b = P(4);
    float* S = F(5);
    const int32_t* n = I(6);
    int32_t B = 4, K = 7, H = 2, Dk = 128, Dv = 128;
    int dt = KDA_BF16;
    int32_t upd = 1;
    void* o = P(7);
    int call() const {
        return kda_decode_multi(q, k, v, g, b, S, n, B, K, H, Dk, Dv, (kda_dtype)dt, upd, o,
                                nullptr);
    }
};

struct SnapA {
    ChunkA c;
    int32_t interval = 512;
    const int32_t* scu = I(9);
    int64_t n_snap = 4;
    float* snap = F(10);
    int call() const {
        return kda_chunk_fwd_snap(c.q, c.k, c.v, c.g, c.b, c.h0, c.cu, c.N, c.T, c.H, c.Dk, c.Dv,
                                  (kda_dtype)c.dt, c.o, c.hT, interval, scu, n_snap, snap,
                                  nullptr, 0, nullptr);
    }
};

struct BwdA {
    void *q = P(0), *k = P(1), *v = P(2), *g = P(3), *b = P(4);
    float* h0 = F(5);
    const int32_t* cu = nullptr;
    int32_t N = 1;
    int64_t T = 64;
    int32_t H = 2, Dk = 128, Dv = 128;
    int dt = KDA_BF16;
    void* dout = P(6);
    float* dhT = F(7);
    void *dq = P(8), *dk = P(9), *dv = P(10), *dg = P(11), *db = P(12);
    float* dh0 = F(13);
    void* ws = P(14);
    size_t wsb = 0;
    bool auto_ws = true;
    int call() const {
        const size_t need =
            auto_ws ? kda_chunk_bwd_workspace_size(T, N, H, Dk, Dv, (kda_dtype)dt) : wsb;
        return kda_chunk_bwd(q, k, v, g, b, h0, cu, N, T, H, Dk, Dv, (kda_dtype)dt, dout, dhT,
                             dq, dk, dv, dg, db, dh0, ws, need, nullptr);
    }
};

struct SegA {
    void *q = P(0), *k = P(1), *v = P(2), *g = P(3), *b = P(4);
    const int32_t* cu = I(6);
    int32_t N = 3;
    int64_t T = 600;
    int32_t H = 2, Dk = 128, Dv = 128;
    int dt = KDA_BF16;
    float *M = F(7), *B = F(8);
    int call() const {
        return kda_segment_summary(q, k, v, g, b, cu, N, T, H, Dk, Dv, (kda_dtype)dt, M, B,
                                   nullptr, 0, nullptr);
    }
};

struct ScanA {
    float *M = F(0), *B = F(1), *h0 = F(2);
    int32_t R = 4, H = 2, Dk = 128, Dv = 128;
    float *S = F(3), *Fin = F(4);
    int call() const { return kda_segment_scan(M, B, h0, R, H, Dk, Dv, S, Fin, nullptr); }
};

struct ProA {
    void *xq = P(0), *xk = P(1), *xv = P(2), *a = P(3), *b = P(4);
    float *w = F(5), *bias = F(6);
    const int32_t* cu = I(7);
    int32_t N = 2;
    int64_t T = 100;
    int32_t H = 3, D = 128;
    int dt = KDA_BF16;
    void *si = P(8), *so = P(9);
    float eps = 1e-6f;
    void *q = P(10), *k = P(11), *v = P(12), *la = P(13), *beta = P(14);
    int call() const {
        return kda_prologue(xq, xk, xv, a, b, w, bias, cu, N, T, H, D, (kda_dtype)dt, si, so, eps,
                            q, k, v, la, beta, nullptr);
    }
};

struct EpiA {
    void *o = P(0), *g = P(1);
    float* w = F(2);
    int64_t T = 100;
    int32_t H = 3, D = 128;
    int dt = KDA_BF16;
    float eps = 1e-5f;
    void* y = P(3);
    int call() const {
        return kda_epilogue(o, g, w, T, H, D, (kda_dtype)dt, eps, y, nullptr);
    }
};

template <typename A>
void case_(const char* what, int want, const std::function<void(A&)>& edit) {
    A a;
    edit(a);
    expect(what, a.call(), want);
}

const std::vector<int64_t> kInts = {INT32_MIN, -129, -1, 0, 1, 2, 15, 16, 17, 32, 127, 128, 129,
                                    4096, 65536, 65537, 1 << 24, INT32_MAX - 1, INT32_MAX};
const std::vector<int64_t> kLongs = {INT64_MIN, -1, 0, 1, 15, 16, 17, 4096, int64_t(1) << 31,
                                     int64_t(1) << 40, int64_t(1) << 50, int64_t(1) << 60,
                                     INT64_MAX};

template <typename A>
void sweep32(const char* what, int32_t A::*field) {
    for (int64_t x : kInts) {
        A a;
        a.*field = (int32_t)x;
        expect_valid(what, a.call());
    }
}
template <typename A>
void sweep64(const char* what, int64_t A::*field) {
    for (int64_t x : kLongs) {
        A a;
        a.*field = x;
        expect_valid(what, a.call());
    }
}

}  // namespace

int main() {
    // ---- part 1: documented status codes ----
    expect("valid chunk", ChunkA().call(), KDA_ERR_DEVICE);
    case_<ChunkA>("chunk dtype", KDA_ERR_BAD_DTYPE, [](ChunkA& a) { a.dt = 2; });
    case_<ChunkA>("chunk Dk", KDA_ERR_BAD_SHAPE, [](ChunkA& a) { a.Dk = 64; });
    case_<ChunkA>("chunk H max", KDA_ERR_BAD_SHAPE, [](ChunkA& a) { a.H = KDA_MAX_HEADS + 1; });
    case_<ChunkA>("chunk N without cu", KDA_ERR_BAD_SHAPE, [](ChunkA& a) { a.N = 2; a.cu = nullptr; });
    case_<ChunkA>("chunk length", KDA_ERR_BAD_SHAPE, [](ChunkA& a) { a.chunk = 48; });
    case_<ChunkA>("chunk split", KDA_ERR_BAD_SHAPE, [](ChunkA& a) { a.split = 3; });
    case_<ChunkA>("chunk null q", KDA_ERR_NULL_ARG, [](ChunkA& a) { a.q = nullptr; });
    case_<ChunkA>("chunk null o", KDA_ERR_NULL_ARG, [](ChunkA& a) { a.o = nullptr; });
    case_<ChunkA>("chunk misaligned q", KDA_ERR_MISALIGNED, [](ChunkA& a) { a.q = P(0, 8); });
    case_<ChunkA>("chunk misaligned cu", KDA_ERR_MISALIGNED, [](ChunkA& a) { a.cu = I(6, 2); });
    case_<ChunkA>("chunk beta element-aligned", KDA_ERR_ALIAS,
                  [](ChunkA& a) { a.b = P(4, 6); a.o = P(4); });
    case_<ChunkA>("chunk o inside q", KDA_ERR_ALIAS, [](ChunkA& a) { a.o = P(0, 64); });
    case_<ChunkA>("chunk h_T on h0", KDA_ERR_ALIAS, [](ChunkA& a) { a.hT = F(5); });
    case_<ChunkA>("chunk empty", KDA_ERR_DEVICE,
                  [](ChunkA& a) { a.T = 0; a.q = a.k = a.v = a.g = a.b = a.o = nullptr; });

    expect("valid decode", DecodeA().call(), KDA_ERR_DEVICE);
    case_<DecodeA>("decode H max", KDA_ERR_BAD_SHAPE, [](DecodeA& a) { a.H = KDA_MAX_HEADS + 1; });
    case_<DecodeA>("decode B < 0", KDA_ERR_BAD_SHAPE, [](DecodeA& a) { a.B = -1; });
    case_<DecodeA>("decode null S", KDA_ERR_NULL_ARG, [](DecodeA& a) { a.S = nullptr; });
    case_<DecodeA>("decode misaligned S", KDA_ERR_MISALIGNED, [](DecodeA& a) { a.S = F(5, 8); });
    case_<DecodeA>("decode o inside S", KDA_ERR_ALIAS, [](DecodeA& a) { a.o = P(5, 4096); });
    case_<DecodeA>("decode empty", KDA_OK, [](DecodeA& a) {
        a.B = 0;
        a.q = a.k = a.v = a.g = a.b = a.o = nullptr;
        a.S = nullptr;
    });

    expect("valid multi", MultiA().call(), KDA_ERR_DEVICE);
    case_<MultiA>("multi K = 0", KDA_ERR_BAD_SHAPE, [](MultiA& a) { a.K = 0; });
    case_<MultiA>("multi o on n_tok", KDA_ERR_ALIAS, [](MultiA& a) { a.o = P(6); });
    case_<MultiA>("multi misaligned n_tok", KDA_ERR_MISALIGNED, [](MultiA& a) { a.n = I(6, 2); });

    expect("valid snap", SnapA().call(), KDA_ERR_DEVICE);
    case_<SnapA>("snap interval", KDA_ERR_BAD_SHAPE, [](SnapA& a) { a.interval = 100; });
    case_<SnapA>("snap null", KDA_ERR_NULL_ARG, [](SnapA& a) { a.snap = nullptr; });
    case_<SnapA>("snap on h_T", KDA_ERR_ALIAS, [](SnapA& a) { a.snap = F(8); });
    case_<SnapA>("snap n_snap < 0", KDA_ERR_BAD_SHAPE, [](SnapA& a) { a.n_snap = -1; });

    expect("valid bwd", BwdA().call(), KDA_ERR_DEVICE);
    case_<BwdA>("bwd no workspace", KDA_ERR_WORKSPACE, [](BwdA& a) { a.ws = nullptr; });
    case_<BwdA>("bwd short workspace", KDA_ERR_WORKSPACE,
                [](BwdA& a) { a.auto_ws = false; a.wsb = 1024; });
    case_<BwdA>("bwd null dout", KDA_ERR_NULL_ARG, [](BwdA& a) { a.dout = nullptr; });
    case_<BwdA>("bwd two gradients", KDA_ERR_ALIAS, [](BwdA& a) { a.dk = P(8); });
    case_<BwdA>("bwd workspace over q", KDA_ERR_ALIAS, [](BwdA& a) { a.ws = P(0); });

    // the allocation-free backward: same validation, then its size limit
    {
        BwdA a;
        expect("noalloc valid", kda_chunk_bwd_noalloc(a.q, a.k, a.v, a.g, a.b, a.h0, a.cu, a.N, a.T,
                                                      a.H, a.Dk, a.Dv, KDA_BF16, a.dout, a.dhT,
                                                      a.dq, a.dk, a.dv, a.dg, a.db, a.dh0,
                                                      nullptr),
               KDA_ERR_DEVICE);
        expect("noalloc oversize", kda_chunk_bwd_noalloc(a.q, a.k, a.v, a.g, a.b, a.h0, a.cu, a.N,
                                                         4096, 96, a.Dk, a.Dv, KDA_BF16, a.dout,
                                                         a.dhT, a.dq, a.dk, a.dv, a.dg, a.db,
                                                         a.dh0, nullptr),
               KDA_ERR_WORKSPACE);
        expect("noalloc alias", kda_chunk_bwd_noalloc(a.q, a.k, a.v, a.g, a.b, a.h0, a.cu, a.N, a.T,
                                                      a.H, a.Dk, a.Dv, KDA_BF16, a.dout, a.dhT,
                                                      a.dq, a.dq, a.dv, a.dg, a.db, a.dh0,
                                                      nullptr),
               KDA_ERR_ALIAS);
        for (int64_t T : kLongs)
            expect_valid("noalloc T", kda_chunk_bwd_noalloc(a.q, a.k, a.v, a.g, a.b, a.h0, a.cu,
                                                            a.N, T, a.H, a.Dk, a.Dv, KDA_BF16,
                                                            a.dout, a.dhT, a.dq, a.dk, a.dv, a.dg,
                                                            a.db, a.dh0, nullptr));
    }

    expect("valid summary", SegA().call(), KDA_ERR_DEVICE);
    case_<SegA>("summary none", KDA_ERR_NULL_ARG, [](SegA& a) { a.M = a.B = nullptr; });
    case_<SegA>("summary M on B", KDA_ERR_ALIAS, [](SegA& a) { a.M = F(8); });
    expect("valid scan", ScanA().call(), KDA_ERR_DEVICE);
    case_<ScanA>("scan S on M", KDA_ERR_ALIAS, [](ScanA& a) { a.S = F(0); });
    case_<ScanA>("scan R < 0", KDA_ERR_BAD_SHAPE, [](ScanA& a) { a.R = -1; });

    expect("valid prologue", ProA().call(), KDA_ERR_DEVICE);
    case_<ProA>("prologue eps nan", KDA_ERR_BAD_SHAPE, [](ProA& a) { a.eps = 0.f / 0.f; });
    case_<ProA>("prologue history alias", KDA_ERR_ALIAS, [](ProA& a) { a.so = P(8); });
    case_<ProA>("prologue misaligned beta", KDA_ERR_MISALIGNED, [](ProA& a) { a.beta = P(14, 1); });
    expect("valid epilogue", EpiA().call(), KDA_ERR_DEVICE);
    case_<EpiA>("epilogue in place", KDA_ERR_DEVICE, [](EpiA& a) { a.y = P(0); });
    case_<EpiA>("epilogue partial overlap", KDA_ERR_ALIAS, [](EpiA& a) { a.y = P(0, 256); });

    // ---- part 2: every integer argument over extreme values ----
    sweep32<ChunkA>("chunk N", &ChunkA::N);
    sweep32<ChunkA>("chunk H", &ChunkA::H);
    sweep32<ChunkA>("chunk Dk", &ChunkA::Dk);
    sweep32<ChunkA>("chunk Dv", &ChunkA::Dv);
    sweep32<ChunkA>("chunk chunk", &ChunkA::chunk);
    sweep32<ChunkA>("chunk split", &ChunkA::split);
    sweep64<ChunkA>("chunk T", &ChunkA::T);
    sweep32<DecodeA>("decode B", &DecodeA::B);
    sweep32<DecodeA>("decode H", &DecodeA::H);
    sweep32<MultiA>("multi B", &MultiA::B);
    sweep32<MultiA>("multi K", &MultiA::K);
    sweep32<MultiA>("multi H", &MultiA::H);
    sweep32<SnapA>("snap interval", &SnapA::interval);
    sweep64<SnapA>("snap n_snap", &SnapA::n_snap);
    sweep32<BwdA>("bwd N", &BwdA::N);
    sweep32<BwdA>("bwd H", &BwdA::H);
    sweep64<BwdA>("bwd T", &BwdA::T);
    sweep32<SegA>("summary N", &SegA::N);
    sweep32<SegA>("summary H", &SegA::H);
    sweep64<SegA>("summary T", &SegA::T);
    sweep32<ScanA>("scan R", &ScanA::R);
    sweep32<ScanA>("scan H", &ScanA::H);
    sweep32<ProA>("prologue N", &ProA::N);
    sweep32<ProA>("prologue H", &ProA::H);
    sweep64<ProA>("prologue T", &ProA::T);
    sweep32<EpiA>("epilogue H", &EpiA::H);
    sweep64<EpiA>("epilogue T", &EpiA::T);
    // the size queries never fail; only undefined behaviour in them would show here
    volatile size_t sink = 0;
    for (int64_t T : kLongs)
        for (int64_t N : kInts)
            for (int64_t H : {int64_t(1), int64_t(96), int64_t(65536), int64_t(INT32_MAX)}) {
                sink = sink + kda_chunk_bwd_workspace_size(T, (int32_t)N, (int32_t)H, 128, 128,
                                                           KDA_BF16);
                sink = sink + kda_chunk_fwd_workspace_size(T, (int32_t)N, (int32_t)H, 128, 128,
                                                           KDA_F32);
            }
    for (int s = -2; s < 10; ++s)
        if (kda_status_str((kda_status)s)[0] != 'K') {
            fprintf(stderr, "FAIL: status string %d\n", s);
            ++failures;
        }

    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("abi driver: all checks passed\n");
    return 0;
}
