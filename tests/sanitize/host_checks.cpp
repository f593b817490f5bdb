// Drives the host-side layer of libvimscan.so (csrc/host.cpp: argument
// validation, overflow guards, workspace sizes) with ordinary and extreme
// arguments. Built with g++ under -fsanitize=address,undefined by
// tests/test_sanitizers.py: any out-of-bounds access, signed overflow or other
// undefined behaviour aborts the run; a wrong status code fails a CHECK.
// Test infrastructure; nothing here is part of the library.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>

#include "vs_internal.h"

#define CHECK(cond)                                                               \
    do {                                                                          \
        if (!(cond)) {                                                            \
            std::fprintf(stderr, "CHECK failed at line %d: %s\n", __LINE__, #cond); \
            std::exit(1);                                                         \
        }                                                                         \
    } while (0)

namespace {

constexpr int64_t kMax = std::numeric_limits<int64_t>::max();

void* fake(int i) { return reinterpret_cast<void*>((uintptr_t(1) << 40) + uintptr_t(i) * (uintptr_t(1) << 33)); }

vs::Call vim_call(int64_t batch, int64_t dim, int64_t L, int dtype = VS_BF16) {
    vs::Call c{vs::kModeVim, batch, dim, 16, L, 0, 0, dtype, 0,
               fake(0), fake(1), fake(2), fake(3), fake(4),
               static_cast<const float*>(fake(5)), static_cast<const float*>(fake(6)),
               static_cast<const float*>(fake(7)), VS_FLAG_SOFTPLUS, fake(8), fake(9),
               size_t(1) << 40, nullptr};
    return c;
}

void product_guard() {
    CHECK(vs::product_below(2, 3, 4, 25));
    CHECK(!vs::product_below(5, 5, 1, 25));
    CHECK(!vs::product_below(kMax, kMax, kMax, int64_t(1) << 30));
    CHECK(vs::product_below(int64_t(1) << 29, int64_t(1) << 29, 2, kMax));    // 2^59 fits
    CHECK(!vs::product_below(int64_t(1) << 32, int64_t(1) << 32, 2, kMax));   // 2^65 would wrap
    CHECK(vs::product_below(int64_t(1) << 20, int64_t(1) << 20, int64_t(1) << 20, kMax));
    CHECK(!vs::product_below(int64_t(1) << 31, int64_t(1) << 31, int64_t(1) << 31, kMax));
    CHECK(!vs::product_below(0, 5, 5, 100));
    CHECK(!vs::product_below(-3, 5, 5, 100));
}

void overlap_at_the_top() {
    const void* top = reinterpret_cast<const void*>(~uintptr_t(0) - 15);
    const void* low = reinterpret_cast<const void*>(uintptr_t(64));
    CHECK(vs::overlaps(top, 16, top, 16));
    CHECK(!vs::overlaps(top, 16, low, 16));
    CHECK(!vs::overlaps(low, 16, top, 16));
    CHECK(vs::overlaps(low, 100, reinterpret_cast<const void*>(uintptr_t(127)), 1));
    CHECK(!vs::overlaps(low, 64, reinterpret_cast<const void*>(uintptr_t(128)), 1));
}

void scan_validation() {
    vs::Call ok = vim_call(8, 768, 4097);
    CHECK(vs::prepare(ok) == VS_OK);
    // sizes whose products overflow int64 unless they are bounded first
    for (int64_t big : {int64_t(1) << 30, (int64_t(1) << 30) + 1, kMax}) {
        vs::Call c = vim_call(65535, big, big);
        const int rc = vs::prepare(c);
        CHECK(rc == VS_ERR_SHAPE || rc == VS_ERR_UNSUPPORTED);
        c = vim_call(65535, 1 << 20, 1 << 20);
        CHECK(vs::prepare(c) == VS_ERR_UNSUPPORTED);
        c = vim_call(kMax, 8, 8);
        CHECK(vs::prepare(c) == VS_ERR_SHAPE);
    }
    vs::Call neg = vim_call(-1, 8, 8);
    CHECK(vs::prepare(neg) == VS_ERR_SHAPE);
    vs::Call flags = vim_call(2, 8, 8);
    flags.softplus = 4;
    CHECK(vs::prepare(flags) == VS_ERR_UNSUPPORTED);
    vs::Call chunks = vim_call(2, 8, 8);
    chunks.chunks = -1;
    CHECK(vs::prepare(chunks) == VS_ERR_SHAPE);
    vs::Call conv = vim_call(2, 8, 8);
    conv.conv = true;
    CHECK(vs::prepare(conv) == VS_ERR_NULL);
    vs::Call alias = vim_call(2, 8, 8);
    alias.y = fake(0);   // the address of u
    CHECK(vs::prepare(alias) == VS_ERR_ALIAS);
    vs::Call grid = vim_call(2, 8, 35);
    grid.mode = vs::kModeCross4;
    grid.H = 5;
    grid.W = 7;
    CHECK(vs::prepare(grid) == VS_OK);
    grid.W = 8;
    CHECK(vs::prepare(grid) == VS_ERR_SHAPE);
    CHECK(!vs::grid_ok(kMax, 2));
    CHECK(!vs::grid_ok(0, 2));
    CHECK(vs::grid_ok(1 << 20, 1));
}

void workspace_sizes() {
    CHECK(vs::scan_ws_bytes(VS_OP_VIM_BIDIR, 8, 768, 4097, VS_BF16) == size_t(8) * 768 * 4097 * 4);
    CHECK(vs::scan_ws_bytes(VS_OP_VIM_BIDIR, kMax, kMax, kMax, VS_BF16) == 0);
    CHECK(vs::scan_ws_bytes(VS_OP_CROSS4, 65535, 1 << 20, 1 << 20, VS_F32) == 0);
    CHECK(vs::scan_ws_bytes(VS_OP_VIM_GRAD, kMax, 2, 2, VS_BF16) == 0);
    CHECK(vs::scan_ws_bytes(VS_OP_VIM_GRAD, 8, 768, 4097, VS_BF16) > size_t(8) * 768 * 4097 * 12);
    size_t offs[6];
    const size_t g = vs::grad_ws_bytes(1, 1, 1, offs);
    CHECK(offs[0] == 0 && offs[4] < offs[5] && offs[5] < g && g % 256 == 0);
    // the per-batch parameter sums hold 2 x dim x (dstate + 2) floats per
    // batch row for the largest dstate
    const size_t g2 = vs::grad_ws_bytes(3, 5, 7, offs);
    CHECK(g2 - offs[5] >= size_t(4) * 3 * 2 * 5 * (VS_MAX_DSTATE + 2));
    // the saved part and the rest add up to the whole, at every size the
    // entry points accept, the largest included
    const int64_t dims[][3] = {{1, 1, 1}, {8, 768, 4097}, {1, 1, int64_t(1) << 26}, {65535, 16, 1023}};
    for (const auto& d : dims) {
        const size_t whole = vs::scan_ws_bytes(VS_OP_VIM_GRAD, d[0], d[1], d[2], VS_BF16);
        const size_t sv = vs::scan_ws_bytes(VS_OP_VIM_SAVED, d[0], d[1], d[2], VS_BF16);
        const size_t rest = vs::scan_ws_bytes(VS_OP_VIM_GRAD_SAVED, d[0], d[1], d[2], VS_BF16);
        CHECK(whole > 0 && sv > 0 && rest > 0 && sv + rest == whole);
        CHECK(sv >= size_t(4) * d[0] * d[1] * d[2]);
    }
    CHECK(vs::scan_ws_bytes(VS_OP_VIM_SAVED, kMax, 2, 2, VS_BF16) == 0);
    CHECK(vs::scan_ws_bytes(7, 8, 768, 4097, VS_BF16) == 0);
}

void grad_validation() {
    vs::GradCall g{8, 768, 16, 4097, VS_BF16, fake(0), fake(1), fake(2), fake(3), fake(4),
                   static_cast<const float*>(fake(5)), static_cast<const float*>(fake(6)),
                   static_cast<const float*>(fake(7)), VS_FLAG_SOFTPLUS, fake(8), fake(9),
                   fake(10), fake(11), static_cast<float*>(fake(12)), static_cast<float*>(fake(13)),
                   static_cast<float*>(fake(14)), static_cast<float*>(fake(15)),
                   static_cast<float*>(fake(16)), fake(17), size_t(1) << 40, nullptr};
    CHECK(vs::validate_grad(g) == VS_OK);
    vs::GradCall big = g;
    big.dim = big.L = int64_t(1) << 30;
    CHECK(vs::validate_grad(big) == VS_ERR_UNSUPPORTED);
    big.dim = big.L = kMax;
    CHECK(vs::validate_grad(big) == VS_ERR_SHAPE);
    vs::GradCall alias = g;
    alias.du = alias.dz;
    CHECK(vs::validate_grad(alias) == VS_ERR_ALIAS);
    // reading a saved buffer: it is an input (no output may overlap it),
    // and the workspace is then only the rest
    vs::GradCall sv = g;
    sv.saved = fake(18);
    sv.saved_bytes = size_t(1) << 40;
    sv.ws_bytes = vs::scan_ws_bytes(VS_OP_VIM_GRAD_SAVED, 8, 768, 4097, VS_BF16);
    CHECK(vs::validate_grad(sv) == VS_OK);
    vs::GradCall short_sv = sv;
    short_sv.saved_bytes = vs::scan_ws_bytes(VS_OP_VIM_SAVED, 8, 768, 4097, VS_BF16) - 1;
    CHECK(vs::validate_grad(short_sv) == VS_ERR_WORKSPACE);
    vs::GradCall on_sv = sv;
    on_sv.dB = static_cast<float*>(fake(18));
    CHECK(vs::validate_grad(on_sv) == VS_ERR_ALIAS);
    // the saving forward: the saved buffer stands for the workspace
    vs::Call c{vs::kModeVim, 8, 768, 16, 4097, 0, 0, VS_BF16, 0, fake(0), fake(1), fake(2), fake(3),
               fake(4), static_cast<const float*>(fake(5)), nullptr, nullptr, VS_FLAG_SOFTPLUS,
               fake(9), fake(18), size_t(1) << 40, nullptr};
    c.saved_fwd = true;
    CHECK(vs::prepare(c) == VS_OK);
    vs::Call zoh = c;
    zoh.softplus = VS_FLAG_SOFTPLUS | VS_FLAG_ZOH;
    zoh.saved_fwd = true;
    CHECK(vs::prepare(zoh) == VS_ERR_UNSUPPORTED);
    vs::Call longer = c;
    longer.batch = longer.dim = 1;
    longer.L = (int64_t(1) << 26) + 1;
    CHECK(vs::prepare(longer) == VS_ERR_UNSUPPORTED);
}

void proj_validation() {
    CHECK(vs::validate_x_proj(8, 768, 16, 4097, VS_BF16, fake(0), fake(1), fake(2), fake(3),
                              static_cast<const float*>(fake(4))) == VS_OK);
    CHECK(vs::validate_out_proj(8, 768, 768, 4097, VS_BF16, fake(0), fake(1),
                                static_cast<const float*>(fake(2)), fake(3), fake(3)) == VS_OK);
    CHECK(vs::validate_out_proj(8, kMax, kMax, 4097, VS_BF16, fake(0), fake(1), nullptr, nullptr,
                                fake(3)) == VS_ERR_UNSUPPORTED);
    CHECK(vs::validate_out_proj(65535, 1 << 16, 1 << 16, 1 << 29, VS_BF16, fake(0), fake(1),
                                nullptr, nullptr, fake(3)) == VS_ERR_UNSUPPORTED);
    CHECK(vs::validate_x_proj(8, kMax, 16, kMax, VS_BF16, fake(0), fake(1), fake(2), fake(3),
                              static_cast<const float*>(fake(4))) == VS_ERR_UNSUPPORTED);
    CHECK(vs::validate_dt_proj(8, kMax, 4097, VS_BF16, static_cast<const float*>(fake(0)),
                               static_cast<const float*>(fake(1)), fake(2)) == VS_ERR_UNSUPPORTED);
    CHECK(vs::validate_dt_proj(8, 768, 4097, VS_F32, static_cast<const float*>(fake(0)),
                               static_cast<const float*>(fake(1)), fake(2)) == VS_ERR_UNSUPPORTED);
}

}  // namespace

int main() {
    product_guard();
    overlap_at_the_top();
    scan_validation();
    workspace_sizes();
    grad_validation();
    proj_validation();
    std::printf("host checks ok\n");
    return 0;
}
