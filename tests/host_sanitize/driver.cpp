// Host-only exercise of the C-ABI layer and the pack-table builders, built
// with AddressSanitizer and UndefinedBehaviorSanitizer (see
// tests/test_host_sanitize.py).  The launchers are host stubs that count
// their calls (stubs.cpp), so nothing here touches a GPU.
//
// Checked for every entry point, over seeded random arguments drawn from
// boundary values (null, misaligned and aligned pointers; zero, negative,
// small, power-of-two and extreme sizes; non-finite floats):
//   * a call returns a known status;
//   * a rejected call (any status other than MF_OK and MF_ERR_HIP) launches
//     nothing, and a call that launches reports the launch's result;
//   * the sanitizers see no invalid memory access and no undefined
//     arithmetic (signed overflow, bad shifts, misaligned host accesses) in
//     the argument checks.
// The pack-table builders run over random descriptor lists, valid and not,
// writing into buffers of exactly the reported size.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <random>
#include <vector>

#include "mf.h"

extern long g_launches;

namespace {

int failures = 0;
// Second pass: the pickers favour values a call accepts (aligned non-null
// pointers, typical sizes, finite floats), so that the checks of calls that
// go on to launch run too.
bool g_valid_mode = false;

void fail(const char* what, int status) {
    if (++failures <= 20) std::fprintf(stderr, "FAIL %s: status %d\n", what, status);
}

bool known(int s) { return s <= 0 && s >= -8; }

// Host memory standing in for device buffers: the checks only look at the
// pointer values (alignment, null), never at the memory.
unsigned char* g_buf = nullptr;

struct Rng {
    std::mt19937_64 g;
    explicit Rng(uint64_t seed) : g(seed) {}
    template <typename T>
    T pick(std::initializer_list<T> xs) {
        return *(xs.begin() + g() % xs.size());
    }
    const void* ptr() {
        if (g_valid_mode && g() % 16 != 0) return g_buf + 256 * (g() % 4);
        switch (g() % 6) {
            case 0: return nullptr;
            case 1: return g_buf + 2;      // misaligned for 16 bytes
            case 2: return g_buf + 4;
            default: return g_buf + 256 * (g() % 4);
        }
    }
    void* wptr() { return const_cast<void*>(ptr()); }
    int32_t i32() {
        if (g_valid_mode && g() % 8 != 0) return pick<int32_t>({0, 1, 2, 3, 4, 8, 16, 24, 32, 64, 128, 256, 3072});
        return pick<int32_t>({-1, 0, 1, 2, 3, 7, 8, 16, 32, 63, 64, 65, 96, 128, 129, 256, 4096, 4097, 65536,
                              std::numeric_limits<int32_t>::max(), std::numeric_limits<int32_t>::min()});
    }
    int64_t i64() {
        if (g_valid_mode && g() % 8 != 0) return pick<int64_t>({1, 2, 8, 64, 128, 256, 1024, 3072, 9216});
        return pick<int64_t>({-1, 0, 1, 8, 64, 1000, 3072, 9216, int64_t(1) << 20, int64_t(1) << 31,
                              int64_t(1) << 40, std::numeric_limits<int64_t>::max() / 2,
                              std::numeric_limits<int64_t>::max(), std::numeric_limits<int64_t>::min()});
    }
    size_t sz() {
        if (g_valid_mode && g() % 8 != 0) return size_t(1) << 40;
        return pick<size_t>({0, 1, 255, 4096, 1 << 20, size_t(1) << 40, ~size_t(0)}); }
    float f() {
        if (g_valid_mode && g() % 8 != 0) return pick<float>({1e-6f, 0.0883883f, 0.125f, 1.f, 10000.f});
        return pick<float>({-1.f, 0.f, 1e-6f, 0.0883883f, 1.f, 10000.f, std::nanf(""),
                            std::numeric_limits<float>::infinity()});
    }
    int32_t* i32p() { return static_cast<int32_t*>(wptr()); }
    float* f32p() { return static_cast<float*>(wptr()); }
};

// One fuzzed call: the launch counter must move exactly when the status says
// a launch happened.
template <typename F>
void fuzz(const char* name, uint64_t seed, int n, F call) {
    Rng r(g_valid_mode ? seed + 1000 : seed);
    const long start = g_launches;
    for (int i = 0; i < n; ++i) {
        const long before = g_launches;
        const int s = int(call(r));
        const long launched = g_launches - before;
        if (!known(s)) fail(name, s);
        if (s == MF_ERR_HIP) {
            if (launched == 0) fail(name, s);
        } else if (s != MF_OK) {
            if (launched != 0) fail(name, s);
        }
    }
    if (g_valid_mode) std::printf("  %-32s %6ld launches of %d calls\n", name, g_launches - start, n);
}

void pack_tables() {
    Rng r(7);
    for (int it = 0; it < 4000; ++it) {
        const int n = int(r.g() % 9);
        std::vector<mf_sample_desc> d(static_cast<size_t>(n));
        for (auto& x : d) {
            const bool wild = r.g() % 5 == 0;
            x.text_len = wild ? r.i32() : int32_t(r.g() % 300);
            x.n_frames = wild ? r.i32() : int32_t(1 + r.g() % 3);
            x.grid_h = wild ? r.i32() : int32_t(r.g() % 70);
            x.grid_w = wild ? r.i32() : int32_t(r.g() % 70);
            x.mod_row_text = wild ? r.i32() : int32_t(r.g() % 4);
            x.mod_row_image = wild ? r.i32() : int32_t(r.g() % 4);
        }
        int64_t T = -1;
        const mf_status s = mf_pack_count(d.data(), n, &T);
        if (!known(s)) fail("mf_pack_count", s);
        if (s != MF_OK) continue;
        if (T < 0 || T > (int64_t(1) << 16)) continue;   // keep the buffers small
        std::vector<int32_t> cu(static_cast<size_t>(n) + 1), pos(static_cast<size_t>(3 * T)),
            sid(static_cast<size_t>(T)), mr(static_cast<size_t>(T));
        const mf_status s2 = mf_pack_tables(d.data(), n, cu.data(), pos.data(), sid.data(), mr.data());
        if (s2 != MF_OK) fail("mf_pack_tables", s2);
        // packed CFG rows over random prompt pairs
        if (n >= 2) {
            const int np = n / 2;
            std::vector<int32_t> cond(static_cast<size_t>(np)), uncond(static_cast<size_t>(np));
            for (int p = 0; p < np; ++p) {
                cond[size_t(p)] = r.g() % 7 == 0 ? r.i32() : 2 * p;
                uncond[size_t(p)] = r.g() % 7 == 0 ? r.i32() : 2 * p + 1;
            }
            int64_t NT = -1;
            const mf_status s3 = mf_cfg_pair_count(d.data(), n, cond.data(), uncond.data(), np, &NT);
            if (!known(s3)) fail("mf_cfg_pair_count", s3);
            if (s3 == MF_OK && NT >= 0 && NT <= (int64_t(1) << 16)) {
                std::vector<int32_t> rows(static_cast<size_t>(2 * NT));
                const mf_status s4 = mf_cfg_pair_rows(d.data(), n, cond.data(), uncond.data(), np, rows.data());
                if (s4 != MF_OK) fail("mf_cfg_pair_rows", s4);
            }
        }
    }
    for (int it = 0; it < 2000; ++it) {
        const int n = int(r.g() % 9);
        std::vector<int32_t> lens(static_cast<size_t>(n));
        int64_t T = 0;
        for (auto& L : lens) {
            L = r.g() % 6 == 0 ? r.i32() : int32_t(r.g() % 600);
            T += L > 0 ? L : 0;
        }
        if (T > (int64_t(1) << 16)) continue;
        std::vector<int32_t> cu(static_cast<size_t>(n) + 1), pos(static_cast<size_t>(T) + 1);
        const mf_status s = mf_prompt_tables(lens.data(), n, cu.data(), pos.data());
        if (!known(s)) fail("mf_prompt_tables", s);
    }
}

void abi() {
    const int N = 3000;
    fuzz("mf_modulate_rope", 11, N, [](Rng& r) {
        return mf_modulate_rope(nullptr, r.ptr(), r.ptr(), r.wptr(), r.wptr(), r.i64(), r.i32(), r.i32(), r.i64(),
                                r.i64(), r.ptr(), r.ptr(), r.i32p(), r.i32(), r.i32p(), r.i32(), r.i32(), r.i32(),
                                r.f(), r.f());
    });
    fuzz("mf_varlen_attn_workspace_bytes", 12, N, [](Rng& r) {
        (void)mf_varlen_attn_workspace_bytes(r.i32(), r.i64(), r.i32(), r.i32());
        return MF_OK;
    });
    fuzz("mf_varlen_attn_fwd", 13, N, [](Rng& r) {
        return mf_varlen_attn_fwd(nullptr, r.ptr(), r.ptr(), r.ptr(), r.wptr(), r.f32p(), r.i32p(), r.i32(), r.i32(),
                                  r.i64(), r.i32(), r.i32(), r.i64(), r.i64(), r.f(), r.wptr(), r.sz());
    });
    fuzz("mf_varlen_attn_fwd_noalloc", 14, N, [](Rng& r) {
        return mf_varlen_attn_fwd_noalloc(nullptr, r.ptr(), r.ptr(), r.ptr(), r.wptr(), r.f32p(), r.i32p(), r.i32(),
                                          r.i32(), r.i64(), r.i32(), r.i32(), r.i64(), r.i64(), r.f());
    });
    fuzz("mf_set_attn_fwd_grid", 15, 200, [](Rng& r) {
        const int s = int(mf_set_attn_fwd_grid(r.i32()));
        mf_set_attn_fwd_grid(0);
        return s;
    });
    fuzz("mf_varlen_attn_bwd", 16, N, [](Rng& r) {
        return mf_varlen_attn_bwd(nullptr, r.ptr(), r.ptr(), r.ptr(), r.ptr(), r.ptr(), r.f32p(), r.wptr(), r.wptr(),
                                  r.wptr(), r.i32p(), r.i32(), r.i32(), r.i64(), r.i32(), r.i32(), r.i64(), r.i64(),
                                  r.i64(), r.f(), r.wptr(), r.sz());
    });
    fuzz("mf_modulate_rope_bwd", 17, N, [](Rng& r) {
        return mf_modulate_rope_bwd(nullptr, r.ptr(), r.ptr(), r.i64(), r.ptr(), r.ptr(), r.i64(), r.wptr(), r.wptr(),
                                    r.i64(), r.i64(), r.i32(), r.i32(), r.ptr(), r.i32p(), r.i32(), r.f32p(),
                                    r.f32p(), r.i32p(), r.i32(), r.i32(), r.i32(), r.f(), r.f(), r.wptr(), r.sz());
    });
    fuzz("mf_gated_residual_bwd", 18, N, [](Rng& r) {
        return mf_gated_residual_bwd(nullptr, r.ptr(), r.ptr(), r.ptr(), r.i32p(), r.i32(), r.ptr(), r.ptr(),
                                     r.ptr(), r.wptr(), r.wptr(), r.f32p(), r.f32p(), r.f32p(), r.i64(), r.i32(),
                                     r.f(), r.wptr(), r.sz());
    });
    fuzz("mf_gated_residual", 19, N, [](Rng& r) {
        return mf_gated_residual(nullptr, r.ptr(), r.ptr(), r.wptr(), r.ptr(), r.i32p(), r.i32(), r.ptr(), r.ptr(),
                                 r.wptr(), r.i64(), r.i32(), r.f());
    });
    fuzz("mf_block_qkv", 20, N, [](Rng& r) {
        return mf_block_qkv(nullptr, r.ptr(), r.i64(), r.ptr(), r.wptr(), r.i64(), r.ptr(), r.ptr(), r.i32p(),
                            r.i32(), r.i32p(), r.i64(), r.i32(), r.i32(), r.i32(), r.i32(), r.i32(), r.f(), r.f(),
                            r.wptr(), r.sz());
    });
    fuzz("mf_block_out", 21, N, [](Rng& r) {
        return mf_block_out(nullptr, r.ptr(), r.i64(), r.ptr(), r.ptr(), r.ptr(), r.i32p(), r.i32(), r.wptr(),
                            r.i64(), r.i32());
    });
    fuzz("mf_cfg_euler_step", 22, N, [](Rng& r) {
        return mf_cfg_euler_step(nullptr, r.ptr(), r.i64(), r.i32p(), static_cast<const float*>(r.ptr()), r.f32p(),
                                 r.wptr(), r.i64(), r.i64(), r.i32(), r.f(), r.f(), r.f());
    });
    fuzz("mf_qk_norm_rope", 23, N, [](Rng& r) {
        return mf_qk_norm_rope(nullptr, r.ptr(), r.i64(), r.ptr(), r.i64(), r.wptr(), r.i64(), r.wptr(), r.i64(),
                               r.ptr(), r.ptr(), r.i32p(), r.i64(), r.i32(), r.i32(), r.i32(), r.f(), r.f());
    });
    fuzz("mf_varlen_attn_causal_fwd", 24, N, [](Rng& r) {
        return mf_varlen_attn_causal_fwd(nullptr, r.ptr(), r.i64(), r.ptr(), r.ptr(), r.i64(), r.wptr(), r.i64(),
                                         r.f32p(), r.i32p(), r.i32(), r.i64(), r.i32(), r.i32(), r.i32(), r.f(),
                                         r.wptr(), r.sz());
    });
    fuzz("workspace queries", 25, N, [](Rng& r) {
        (void)mf_varlen_attn_bwd_workspace_bytes(r.i32(), r.i64(), r.i32(), r.i32());
        (void)mf_modulate_rope_bwd_workspace_bytes(r.i64(), r.i32(), r.i32());
        (void)mf_gated_residual_bwd_workspace_bytes(r.i64(), r.i32());
        (void)mf_block_qkv_workspace_bytes(r.i64(), r.i32(), r.i32());
        (void)mf_varlen_attn_causal_workspace_bytes(r.i32(), r.i64());
        return MF_OK;
    });
    for (int s = -10; s <= 2; ++s)
        if (mf_status_string(mf_status(s)) == nullptr) fail("mf_status_string", s);
}

// Explicit valid calls: each must pass every check and reach its launcher
// (which fails, as on a machine without a GPU).
void valid_calls() {
    unsigned char* b = g_buf;
    int32_t* ip = reinterpret_cast<int32_t*>(g_buf);
    float* fp = reinterpret_cast<float*>(g_buf);
    auto expect_launch = [](const char* name, mf_status s) {
        if (s != MF_ERR_HIP) fail(name, s);
    };
    for (int64_t T : {1, 63, 64, 65, 4352}) {
        for (int32_t D : {64, 128}) {
            const int32_t H = 3;
            const int64_t ld = int64_t(H) * D;
            expect_launch("valid mf_modulate_rope",
                          mf_modulate_rope(nullptr, b, b, b, b, T, H, D, ld, ld, b, b, ip, 2, ip, 0, D / 2, D / 2,
                                           10000.f, 1e-6f));
            expect_launch("valid mf_modulate_rope (RoPE only)",
                          mf_modulate_rope(nullptr, b, b, b, b, T, H, D, ld, ld, nullptr, nullptr, nullptr, 0, ip,
                                           D / 4, D / 4 + (D / 4) % 2, D / 2 - (D / 4) % 2, 10000.f, 1e-6f));
            expect_launch("valid mf_varlen_attn_fwd",
                          mf_varlen_attn_fwd(nullptr, b, b, b, b, fp, ip, 1, int32_t(T), T, H, D, 3 * ld, ld,
                                             0.125f, b, size_t(1) << 40));
            expect_launch("valid mf_varlen_attn_fwd_noalloc",
                          mf_varlen_attn_fwd_noalloc(nullptr, b, b, b, b, fp, ip, 1, int32_t(T), T, H, D, ld, ld,
                                                     0.125f));
            expect_launch("valid mf_varlen_attn_bwd",
                          mf_varlen_attn_bwd(nullptr, b, b, b, b, b, fp, b, b, b, ip, 1, int32_t(T), T, H, D, ld,
                                             ld, ld, 0.125f, b, size_t(1) << 40));
            expect_launch("valid mf_modulate_rope_bwd",
                          mf_modulate_rope_bwd(nullptr, b, b, ld, b, b, ld, b, b, ld, T, H, D, b, ip, 2, fp, fp,
                                               ip, 0, D / 2, D / 2, 10000.f, 1e-6f, b, size_t(1) << 40));
            expect_launch("valid mf_qk_norm_rope",
                          mf_qk_norm_rope(nullptr, b, ld, b, D, b, ld, b, D, b, b, ip, T, H, 1, D, 10000.f, 1e-6f));
            expect_launch("valid mf_varlen_attn_causal_fwd",
                          mf_varlen_attn_causal_fwd(nullptr, b, ld, b, b, D, b, ld, fp, ip, 1, T, H, 1, D, 0.125f,
                                                    b, size_t(1) << 40));
        }
        expect_launch("valid mf_block_qkv",
                      mf_block_qkv(nullptr, b, 256, b, b, 768, b, b, ip, 2, ip, T, 2, 128, 0, 64, 64, 10000.f, 1e-6f,
                                   b, size_t(1) << 40));
        expect_launch("valid mf_gated_residual",
                      mf_gated_residual(nullptr, b, b, b, b, ip, 2, b, b, b, T, 256, 1e-6f));
        expect_launch("valid mf_block_out", mf_block_out(nullptr, b, 256, b, b, b, ip, 2, b, T, 256));
    }
}

}  // namespace

int main() {
    g_buf = static_cast<unsigned char*>(std::aligned_alloc(256, 4096));
    pack_tables();
    abi();
    g_valid_mode = true;
    abi();
    valid_calls();
    std::free(g_buf);
    std::printf("host sanitize driver: %d failure(s), %ld stub launches\n", failures, g_launches);
    return failures == 0 ? 0 : 1;
}
