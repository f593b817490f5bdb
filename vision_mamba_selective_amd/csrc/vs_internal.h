// Internal to libvimscan.so: the host-side layer shared by the kernel
// translation units (argument records, validation, workspace layout and the
// per-thread error record). Not part of the C ABI. host.cpp implements it in
// plain C++ (no HIP), so that it also builds on its own, for instance under
// the address and undefined-behaviour sanitizers.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "vimscan.h"

namespace __attribute__((visibility("hidden"))) vs {

constexpr int kBlockTok = 16;       // tokens per block step of the scan kernels
constexpr int kRowLanes = 16;       // one recurrence per 16-lane row
constexpr int kTileTok = 32;        // tokens per B/C staging tile of the forward scan
constexpr int kBcChunk = 1024;      // gradient: floats per workgroup and block of dB/dC sums
constexpr int64_t kNumCUs = 256;
constexpr int64_t kMaxElems = int64_t(1) << 30;   // per tensor (32-bit byte offsets)
constexpr int64_t kGradMaxL = int64_t(1) << 26;   // gradient descriptors span 2 L x 4 B

enum Mode { kMode1D = 0, kModeVim = 1, kModeCross4 = 2 };

constexpr int kCrossChPerWg = 4;             // cross-scan: channels per workgroup
constexpr int64_t kGridLdsBytes = 8 << 10;   // cross-scan: LDS for the column orders' u and delta
// The cross-scan stages a workgroup's u and delta grids in LDS, in
// column-major order, when they take at most kGridLdsBytes (kCrossChPerWg
// channels x 2 tensors x L entries: fp32 grids up to 256 tokens, bf16 up to
// 512). Beyond that the LDS costs workgroups per CU (the B/C tiles already
// take 36 KB) and the transposed copies in the workspace are faster.
inline bool cross4_grid_in_lds(int64_t L, int dtype) {
    return L >= 1 && 2 * kCrossChPerWg * L * (dtype == VS_BF16 ? 2 : 4) <= kGridLdsBytes;
}

constexpr int kVimChPerWg = 8;                // Vim scan: channels per workgroup
constexpr int kPartLdsGuard = 16;             // Vim: LDS entries before and after the partial sums
constexpr int64_t kPartLdsBytes = 8 << 10;    // Vim: LDS for the partial sums of short sequences
// The Vim scan's two directions hand their partial sums to each other
// through LDS instead of an fp32 buffer in global memory when a workgroup's
// rows fit in kPartLdsBytes: kVimChPerWg channels x Lc entries (Lc the
// longest chunk) and a guard of kPartLdsGuard entries at each end, which
// sequences up to 252 tokens per chunk meet.
inline int64_t vim_partial_lds_bytes(int64_t Lc) { return (kVimChPerWg * Lc + 2 * kPartLdsGuard) * 4; }

// One forward scan call (every scan entry point but the gradient).
struct Call {
    int mode;
    int64_t batch, dim, dstate, L;
    int H, W;
    int dtype;
    int reverse;
    const void *u, *delta, *z, *B, *C;
    const float *A, *Dskip, *dt_bias;
    int softplus;                   // flags word on entry, VS_FLAG_SOFTPLUS bit after normalise()
    void* y;
    void* ws;
    size_t ws_bytes;
    void* stream;
    bool conv = false;              // the Vim front-end entry point (conv_w required)
    const float* conv_w = nullptr;  // Vim front end (u then holds x)
    const float* conv_b = nullptr;
    bool per_dir = false;           // Vim: u, delta [2][batch][dim][L]; B, C [batch][2][N][L]
    bool zoh = false;               // exact zero-order-hold B_bar
    int chunks = 0;                 // Vim: chunks per sequence (0: the library's choice)
    bool ws_internal = false;       // the workspace is the library's own (ws_bytes = its capacity)
    bool saved_fwd = false;         // vim_scan_bidir_fwd_saved: ws is the saved-state buffer
};

struct GradCall {
    int64_t batch, dim, dstate, L;
    int dtype;
    const void *u, *delta, *z, *B, *C;
    const float *A, *Dskip, *dt_bias;
    int softplus;
    const void* dy;
    void *du, *ddelta, *dz;
    float *dB, *dC, *dA, *dD, *dbias;
    void* ws;
    size_t ws_bytes;
    void* stream;
    const void* saved = nullptr;    // vim_scan_bidir_grad_saved: the forward's saved states
    size_t saved_bytes = 0;
};

// error record of the calling thread (vs_last_error)
int fail(int code, const std::string& msg);
void clear_error();
const char* last_error();

// a*b*c < limit for a, b, c >= 1, decided without forming a product that
// could overflow
bool product_below(int64_t a, int64_t b, int64_t c, int64_t limit);
bool overlaps(const void* a, size_t na, const void* b, size_t nb);
bool aligned(const void* p, size_t al);

int64_t ndirs(int mode);
// the VMamba grid: H and W in 1..2^20 (so H*W stays in range)
inline bool grid_ok(int64_t H, int64_t W) {
    return H >= 1 && W >= 1 && H <= (int64_t(1) << 20) && W <= (int64_t(1) << 20);
}
// splits the flags word, then checks every argument; VS_OK or a status code
// (with the message recorded). Nothing here touches the HIP runtime.
int prepare(Call& c);
size_t scan_ws_bytes(int op, int64_t batch, int64_t dim, int64_t seqlen, int dtype);

int grad_channels(int64_t batch, int64_t dim);
// the gradient's buffers: the saved part [s][checkpoints] (written by the
// forward pass) and the rest [du partials][ddelta partials][dB/dC chunks]
// [per-batch dA, dD, dt_bias]; the full workspace is the two back to back
size_t grad_saved_bytes(int64_t batch, int64_t dim, int64_t L, size_t offs[2]);
size_t grad_rest_bytes(int64_t batch, int64_t dim, int64_t L, size_t offs[4]);
size_t grad_ws_bytes(int64_t batch, int64_t dim, int64_t L, size_t offs[6]);
int validate_grad(const GradCall& g);

int validate_x_proj(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                    const void* u, const void* W, const void* B, const void* C, const float* dt);
int validate_dt_proj(int64_t batch, int64_t dim, int64_t seqlen, int dtype, const float* dt,
                     const float* w, const void* delta);
int validate_out_proj(int64_t batch, int64_t dim_in, int64_t dim_out, int64_t seqlen, int dtype,
                      const void* y, const void* W, const float* bias, const void* residual,
                      const void* out);

}  // namespace vs
