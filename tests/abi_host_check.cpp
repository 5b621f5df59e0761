// Host-side driver for the sanitizer build of the library's argument
// validation (AddressSanitizer and UndefinedBehaviorSanitizer on the host
// code only; no GPU is touched).  Every entry point of include/gdn.h is
// called with arguments that its checks must refuse before any device work
// -- a negative size, an unsupported width, a null or misaligned pointer, a
// work space one byte short -- and the return code and the last-error
// message are checked; every work-space query is evaluated over a grid of
// sizes up to about 2^31 token-heads, so that an overflow in the size
// arithmetic is reported.  Fake device pointers are aligned addresses that
// the checks compare but never dereference.
//
// Test infrastructure: built and run by tests/test_sanitizers.py.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "gdn.h"

static int failures = 0;

static void expect(const char *what, int rc, int want) {
    const char *msg = gdn_last_error();
    if (rc != want) {
        std::fprintf(stderr, "%s: returned %d, expected %d (%s)\n", what, rc, want, msg ? msg : "(null)");
        ++failures;
    } else if (want != GDN_OK && (!msg || !*msg)) {
        std::fprintf(stderr, "%s: no error message\n", what);
        ++failures;
    }
}

// fake device pointers: 256-byte aligned, or misaligned by `off` bytes
static void *dev(int i, int off = 0) { return reinterpret_cast<void *>((uintptr_t)(0x10000000u + 0x100000u * i + off)); }
static float *devf(int i, int off = 0) { return static_cast<float *>(dev(i, off)); }

static void chunk_fwd_checks() {
    const int B = 2, T = 100, H = 3, D = 64;
    const size_t need = gdn_chunk_fwd_workspace_bytes(B, T, H, D, D, 64, GDN_DTYPE_BF16);
    auto call = [&](const void *q, int b, int dk, int chunk, int dtype, size_t ws) {
        return gdn_chunk_fwd(q, dev(2), dev(3), devf(4), devf(5), 0.125f, nullptr, devf(6), dev(7), b, T, H, dk, D,
                             chunk, dtype, GDN_DTYPE_BF16, dev(8), ws, nullptr);
    };
    expect("gdn_chunk_fwd negative B", call(dev(1), -1, D, 64, GDN_DTYPE_BF16, need), GDN_EINVAL);
    expect("gdn_chunk_fwd Dk=20", call(dev(1), B, 20, 64, GDN_DTYPE_BF16, need), GDN_EUNSUPPORTED);
    expect("gdn_chunk_fwd chunk=48", call(dev(1), B, D, 48, GDN_DTYPE_BF16, need), GDN_EUNSUPPORTED);
    expect("gdn_chunk_fwd dtype=7", call(dev(1), B, D, 64, 7, need), GDN_EINVAL);
    expect("gdn_chunk_fwd null q", call(nullptr, B, D, 64, GDN_DTYPE_BF16, need), GDN_EINVAL);
    expect("gdn_chunk_fwd misaligned q", call(dev(1, 2), B, D, 64, GDN_DTYPE_BF16, need), GDN_EINVAL);
    expect("gdn_chunk_fwd short workspace", call(dev(1), B, D, 64, GDN_DTYPE_BF16, need - 1), GDN_EWORKSPACE);
    expect("gdn_chunk_fwd B=0", call(nullptr, 0, D, 64, GDN_DTYPE_BF16, 0), GDN_OK);

    const float mask[4] = {1.f, 0.f, 1.f, 1.f};
    const size_t dneed = deltaproduct_chunk_fwd_workspace_bytes(B, T, H, 2, 32, D, 32, GDN_DTYPE_BF16);
    auto dcall = [&](const void *q, int r, int dk, const float *m, size_t ws) {
        return deltaproduct_chunk_fwd(q, dev(2), dev(3), devf(4), devf(5), m, r, 0.125f, nullptr, devf(6), dev(7), B,
                                      T, H, dk, D, 32, GDN_DTYPE_BF16, GDN_DTYPE_F32, dev(8), ws, nullptr);
    };
    expect("deltaproduct_chunk_fwd r=3", dcall(dev(1), 3, 32, mask, dneed), GDN_EUNSUPPORTED);
    expect("deltaproduct_chunk_fwd dk=48", dcall(dev(1), 2, 48, mask, dneed), GDN_EUNSUPPORTED);
    expect("deltaproduct_chunk_fwd no mask", dcall(dev(1), 2, 32, nullptr, dneed), GDN_EINVAL);
    expect("deltaproduct_chunk_fwd null q", dcall(nullptr, 2, 32, mask, dneed), GDN_EINVAL);
    expect("deltaproduct_chunk_fwd short workspace", dcall(dev(1), 2, 32, mask, dneed - 1), GDN_EWORKSPACE);
}

static void bwd_checks() {
    const int B = 1, T = 130, H = 2, D = 64;
    const size_t need = gdn_bwd_workspace_bytes(B, T, H, D, D, GDN_DTYPE_BF16);
    auto call = [&](const void *q, int t, int dk, size_t ws) {
        return gdn_bwd(q, dev(2), dev(3), devf(4), devf(5), 0.125f, nullptr, dev(6), nullptr, devf(7), devf(8),
                       devf(9), devf(10), devf(11), nullptr, B, t, H, dk, D, GDN_DTYPE_BF16, dev(12), ws, nullptr);
    };
    expect("gdn_bwd negative T", call(dev(1), -5, D, need), GDN_EINVAL);
    expect("gdn_bwd Dk=24", call(dev(1), T, 24, need), GDN_EUNSUPPORTED);
    expect("gdn_bwd null q", call(nullptr, T, D, need), GDN_EINVAL);
    expect("gdn_bwd misaligned q", call(dev(1, 8), T, D, need), GDN_EINVAL);
    expect("gdn_bwd short workspace", call(dev(1), T, D, need - 1), GDN_EWORKSPACE);

    const float mask[4] = {1.f, 0.f, 1.f, 1.f}, upper[4] = {1.f, 0.5f, 0.f, 1.f};
    const size_t dneed = deltaproduct_bwd_workspace_bytes(B, T, H, 2, D, D, GDN_DTYPE_BF16);
    auto dcall = [&](const void *q, const float *m, int dk, size_t ws) {
        return deltaproduct_bwd(q, dev(2), dev(3), devf(4), devf(5), m, 2, 0.125f, nullptr, dev(6), nullptr, devf(7),
                                devf(8), devf(9), devf(10), devf(11), nullptr, B, T, H, dk, D, GDN_DTYPE_BF16, dev(12),
                                ws, nullptr);
    };
    expect("deltaproduct_bwd upper mask", dcall(dev(1), upper, D, dneed), GDN_EUNSUPPORTED);
    expect("deltaproduct_bwd dk=16", dcall(dev(1), mask, 16, dneed), GDN_EUNSUPPORTED);
    expect("deltaproduct_bwd null q", dcall(nullptr, mask, D, dneed), GDN_EINVAL);
    expect("deltaproduct_bwd short workspace", dcall(dev(1), mask, D, dneed - 1), GDN_EWORKSPACE);
}

static void camera_checks() {
    const int B = 1, H = 2, F = 3, S = 40, D = 64;
    const size_t need = gdn_recurrent_fwd_workspace_bytes(B, H, F, S, D, GDN_DTYPE_BF16);
    auto call = [&](const void *q, int f, int d, size_t ws) {
        return gdn_recurrent_fwd(q, dev(2), dev(3), devf(4), devf(5), 0.125f, nullptr, nullptr, devf(6), B, H, f, S,
                                 d, GDN_DTYPE_BF16, 0, dev(7), ws, nullptr);
    };
    expect("gdn_recurrent_fwd negative F", call(dev(1), -1, D, need), GDN_EINVAL);
    expect("gdn_recurrent_fwd D=40", call(dev(1), F, 40, need), GDN_EUNSUPPORTED);
    expect("gdn_recurrent_fwd null q", call(nullptr, F, D, need), GDN_EINVAL);
    expect("gdn_recurrent_fwd short workspace", call(dev(1), F, D, need - 1), GDN_EWORKSPACE);

    const size_t bneed = gdn_recurrent_bwd_workspace_bytes(B, H, F, S, D, GDN_DTYPE_BF16);
    auto bcall = [&](const void *q, int d, size_t ws) {
        return gdn_recurrent_bwd(q, dev(2), dev(3), devf(4), devf(5), 0.125f, nullptr, devf(6), nullptr, devf(7),
                                 devf(8), devf(9), devf(10), devf(11), nullptr, B, H, F, S, d, GDN_DTYPE_BF16,
                                 dev(12), ws, nullptr);
    };
    expect("gdn_recurrent_bwd D=40", bcall(dev(1), 40, bneed), GDN_EUNSUPPORTED);
    expect("gdn_recurrent_bwd null q", bcall(nullptr, D, bneed), GDN_EINVAL);
    expect("gdn_recurrent_bwd short workspace", bcall(dev(1), D, bneed - 1), GDN_EWORKSPACE);

    const size_t zneed = gdn_recurrent_den_fwd_workspace_bytes(B, H, F, S, D, GDN_DTYPE_BF16);
    auto zcall = [&](const void *q, int d, size_t ws) {
        return gdn_recurrent_den_fwd(q, dev(2), devf(3), devf(4), 0.125f, nullptr, nullptr, devf(5), B, H, F, S, d,
                                     GDN_DTYPE_BF16, 0, dev(6), ws, nullptr);
    };
    expect("gdn_recurrent_den_fwd D=40", zcall(dev(1), 40, zneed), GDN_EUNSUPPORTED);
    expect("gdn_recurrent_den_fwd null q", zcall(nullptr, D, zneed), GDN_EINVAL);
    expect("gdn_recurrent_den_fwd short workspace", zcall(dev(1), D, zneed - 1), GDN_EWORKSPACE);

    const int N = F * S;
    auto pcall = [&](const void *qkv, int d, int dtype) {
        return gdn_prep(qkv, devf(2), devf(3), devf(4), devf(5), devf(6), devf(7), 0.5f, 1e-6f, dev(8), dev(9),
                        dev(10), devf(11), devf(12), nullptr, B, N, H, d, dtype, GDN_DTYPE_BF16, nullptr);
    };
    expect("gdn_prep D=40", pcall(dev(1), 40, GDN_DTYPE_BF16), GDN_EUNSUPPORTED);
    expect("gdn_prep null qkv", pcall(nullptr, D, GDN_DTYPE_BF16), GDN_EINVAL);
    expect("gdn_prep misaligned qkv", pcall(dev(1, 4), D, GDN_DTYPE_BF16), GDN_EINVAL);
    expect("gdn_prep dtype=5", pcall(dev(1), D, 5), GDN_EINVAL);

    const size_t pneed = gdn_prep_bwd_workspace_bytes(B, N, H, D);
    auto qcall = [&](const void *qkv, int d, size_t ws) {
        return gdn_prep_bwd(qkv, devf(2), devf(3), devf(4), devf(5), devf(6), devf(7), 0.5f, 1e-6f, dev(8), dev(9),
                            dev(10), nullptr, nullptr, nullptr, devf(11), devf(12), devf(13), devf(14), devf(15), B, N,
                            H, d, GDN_DTYPE_BF16, GDN_DTYPE_F32, dev(16), ws, nullptr);
    };
    expect("gdn_prep_bwd D=40", qcall(dev(1), 40, pneed), GDN_EUNSUPPORTED);
    expect("gdn_prep_bwd null qkv", qcall(nullptr, D, pneed), GDN_EINVAL);
    if (pneed > 0) expect("gdn_prep_bwd short workspace", qcall(dev(1), D, pneed - 1), GDN_EWORKSPACE);
}

// Work-space queries over sizes up to ~2^31 token-heads: evaluated for their
// arithmetic only (a sanitizer report is the failure); sizes a call refuses
// give 0.
static void workspace_grid() {
    const int Bs[] = {0, 1, 3, 64}, Ts[] = {0, 1, 65, 4096, 1 << 16, 1 << 20}, Hs[] = {1, 16, 64};
    const int Ds[] = {-16, 0, 16, 48, 112, 128, 256, 512}, chunks[] = {0, 16, 32, 48, 64};
    volatile size_t sink = 0;
    for (int B : Bs)
        for (int T : Ts)
            for (int H : Hs) {
                if ((long long)B * T * H > (1ll << 31)) continue;
                for (int D : Ds) {
                    for (int c : chunks)
                        for (int dt = 0; dt < 3; ++dt) {
                            sink = sink + gdn_chunk_fwd_workspace_bytes(B, T, H, D, D, c, dt);
                            sink = sink + deltaproduct_chunk_fwd_workspace_bytes(B, T, H, 2, D / 2, D, c, dt);
                        }
                    for (int dt = 0; dt < 3; ++dt) {
                        sink = sink + gdn_bwd_workspace_bytes(B, T, H, D, D, dt);
                        sink = sink + deltaproduct_bwd_workspace_bytes(B, T, H, 2, D / 2, D, dt);
                        const int S = 1560, F = T / S;
                        sink = sink + gdn_recurrent_fwd_workspace_bytes(B, H, F, S, D, dt);
                        sink = sink + gdn_recurrent_bwd_workspace_bytes(B, H, F, S, D, dt);
                        sink = sink + gdn_recurrent_den_fwd_workspace_bytes(B, H, F, S, D, dt);
                    }
                    sink = sink + gdn_prep_bwd_workspace_bytes(B, T, H, D);
                }
            }
    (void)sink;
}

int main() {
    if (gdn_abi_version() <= 0) {
        std::fprintf(stderr, "gdn_abi_version: %d\n", gdn_abi_version());
        ++failures;
    }
    chunk_fwd_checks();
    bwd_checks();
    camera_checks();
    workspace_grid();
    if (failures) {
        std::fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    std::printf("host validation sanitizer run: all checks passed\n");
    return 0;
}
