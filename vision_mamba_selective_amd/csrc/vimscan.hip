// vimscan.hip -- gfx950 selective-scan kernels and the C ABI of libvimscan.so.
//
// What is computed (see include/vimscan.h for the full contract): the S6
// recurrence of "Vision Mamba Guide: Efficient Bidirectional SSM & VMamba"
// (aifetchly blog), sections "Discretization via Zero-Order Hold" and "The
// Selective State Space (S6) Mechanism", run in the Vim directions of "2. The
// Bidirectional Mamba Block" or the VMamba orders of "1. Cross-Scan
// Traversal", merged as in "Gated State Fusion" / "3. Cross-Merge Reversal".
//
// Mapping onto CDNA4 (one recurrence = one (batch, channel, direction)):
//   * A 16-lane DPP row holds one recurrence; lane n holds state n in a VGPR.
//     A wave64 therefore runs 4 recurrences, which gives the launch
//     batch*dim*ndir*16 lanes: enough waves to fill 256 CUs even at batch 2-8,
//     without splitting the sequence (which would repeat the exp work).
//   * Tokens are processed in blocks of 16. Lane j of a row loads token j of
//     the block (coalesced within the row), computes its delta = softplus(.)
//     and delta*u once, and the row broadcasts them to every state lane with
//     DPP row_newbcast, so no state lane repeats the softplus.
//   * B and C rows of a block are shared by every channel of a batch: the
//     workgroup stages them once per block in LDS (converted to fp32), and each
//     state lane reads its own 16-token window.
//   * The read-out sum over states (y = C . h) is a 16-lane transpose
//     reduction inside the row after each block: lane j ends with token j.
//   * Reverse and column-major orders are index arithmetic on the token
//     address; nothing is flipped or transposed in memory.
//   * Directions that visit a token at different times meet through an fp32
//     partial sum (a workspace, or y itself when y is fp32): the first
//     direction to finish a token stores its contribution, the last one adds
//     it, applies the gate and writes y once.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <type_traits>

#include "vimscan.h"

namespace {

constexpr int kWaveLanes = 64;
constexpr int kRowLanes = 16;       // one recurrence per DPP row
constexpr int kBlockTok = 16;       // tokens per block step
constexpr int kThreads = 256;       // 4 waves per workgroup
constexpr int kTilePad = 20;        // LDS row stride (floats) of a 16-token tile

enum Mode { kMode1D = 0, kModeVim = 1, kModeCross4 = 2 };
enum Order { kFwd = 0, kRev = 1, kCol = 2, kColRev = 3 };

struct ScanArgs {
    const void* u;
    const void* delta;
    const void* z;
    const void* B;
    const void* C;
    const float* A;
    const float* Dskip;
    const float* dt_bias;
    void* y;
    float* partial;     // fp32 partial sums for the merge ([batch][dim][L])
    int64_t dim;
    int64_t L;
    int H;
    int W;
    int dstate;
    int softplus;
    int reverse;        // 1-D mode only
    int nblk;           // ceil(L / 16)
};

// ---------------------------------------------------------------- dtype I/O
__device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
// fp32 -> bf16, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) {
    uint32_t x = __float_as_uint(v);
    uint32_t r = (x & 0x7fffffffu) > 0x7f800000u ? (x | 0x00400000u)
                                                  : x + 0x7fffu + ((x >> 16) & 1u);
    p[i] = static_cast<uint16_t>(r >> 16);
}

// ------------------------------------------------------------- lane moves
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL,
                                                      0xf, 0xf, false));
}
// value of lane I of this 16-lane row, in every lane of the row (row_newbcast)
template <int I>
__device__ __forceinline__ float row_bcast(float v) { return dpp<0x150 + I>(v); }

// value of lane (lane ^ M) within the row
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
    if constexpr (M == 8) return dpp<0x128>(v);                 // row_ror:8
    else if constexpr (M == 2) return dpp<0x4e>(v);             // quad_perm [2,3,0,1]
    else if constexpr (M == 1) return dpp<0xb1>(v);             // quad_perm [1,0,3,2]
    else return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101f));  // xor 4
}

// Transpose-reduce 16 values per lane across the 16 lanes of a row:
// on return c[0] of lane j holds sum over the row's lanes of c[j].
template <int M, int V>
__device__ __forceinline__ void reduce_stage(float (&c)[16], int lane) {
    const bool hi = (lane & M) != 0;
#pragma unroll
    for (int k = 0; k < V / 2; ++k) {
        const float lo_v = c[k], hi_v = c[k + V / 2];
        const float send = hi ? lo_v : hi_v;
        const float keep = hi ? hi_v : lo_v;
        c[k] = keep + xor_lane<M>(send);
    }
}
__device__ __forceinline__ float row_transpose_sum(float (&c)[16], int lane) {
    reduce_stage<8, 16>(c, lane);
    reduce_stage<4, 8>(c, lane);
    reduce_stage<2, 4>(c, lane);
    reduce_stage<1, 2>(c, lane);
    return c[0];
}

// ---------------------------------------------------------------- math
// softplus(x) = log(1 + e^x) in the form that keeps the small result for
// negative x and does not overflow for large x.
__device__ __forceinline__ float softplus_f(float x) {
    return x > 0.f ? x + log1pf(expf(-x)) : log1pf(expf(x));
}
__device__ __forceinline__ float silu_f(float z) { return z / (1.f + expf(-z)); }

__device__ __forceinline__ int64_t visit(int order, int64_t t, int64_t L, int H, int W) {
    switch (order) {
    case kFwd: return t;
    case kRev: return L - 1 - t;
    case kCol: return (t % H) * W + t / H;
    default: { int64_t r = L - 1 - t; return (r % H) * W + r / H; }
    }
}

template <int I>
struct Unroll {
    template <typename F>
    __device__ __forceinline__ static void run(F&& f) {
        Unroll<I - 1>::run(f);
        f(std::integral_constant<int, I - 1>{});
    }
};
template <>
struct Unroll<0> {
    template <typename F>
    __device__ __forceinline__ static void run(F&&) {}
};

// ---------------------------------------------------------------- kernel
// Workgroup = 4 waves = 16 rows. Row roles per mode:
//   1-D   : 16 channels, one direction (args.reverse)
//   Vim   : 8 channels x {forward, backward}
//   Cross4: 4 channels x {row-major, reverse, column-major, reverse}
template <typename T, int MODE>
__global__ __launch_bounds__(kThreads) void rowscan_kernel(const ScanArgs a) {
    constexpr int kDirs = MODE == kModeVim ? 2 : (MODE == kModeCross4 ? 4 : 1);
    constexpr int kChPerWg = 16 / kDirs;
    // B/C tiles: 1-D and Vim share B, C over directions (one tile per distinct
    // token order); Cross4 has per-direction B, C in scan order.
    constexpr int kSides = MODE == kMode1D ? 1 : (MODE == kModeVim ? 2 : 4);
    __shared__ float tile[2][kSides][2][kRowLanes][kTilePad];

    const int tid = threadIdx.x;
    const int lane = tid & (kWaveLanes - 1);
    const int row_in_wg = tid >> 4;           // 0..15
    const int n = lane & (kRowLanes - 1);     // state index, also token slot
    const int dir = row_in_wg % kDirs;
    const int ch = row_in_wg / kDirs;
    const int64_t b = blockIdx.y;
    const int64_t d = static_cast<int64_t>(blockIdx.x) * kChPerWg + ch;
    const bool active = d < a.dim;
    const int64_t L = a.L;
    const T* __restrict__ u = static_cast<const T*>(a.u);
    const T* __restrict__ dl = static_cast<const T*>(a.delta);
    const T* __restrict__ z = static_cast<const T*>(a.z);
    const T* __restrict__ Bp = static_cast<const T*>(a.B);
    const T* __restrict__ Cp = static_cast<const T*>(a.C);
    T* __restrict__ y = static_cast<T*>(a.y);

    int order;
    if (MODE == kModeVim) order = dir;                 // 0 forward, 1 backward
    else if (MODE == kModeCross4) order = dir;         // 0..3
    else order = a.reverse ? kRev : kFwd;

    // per-row parameters
    const int pdir = MODE == kMode1D ? 0 : dir;
    const int64_t prow = static_cast<int64_t>(pdir) * a.dim + (active ? d : 0);
    const float kLog2e = 1.4426950408889634f;
    const float A2 = (active && n < a.dstate) ? a.A[prow * a.dstate + n] * kLog2e : 0.f;
    const float Dk = (active && a.Dskip) ? a.Dskip[prow] : 0.f;
    const float bias = (active && a.dt_bias) ? a.dt_bias[prow] : 0.f;
    const int64_t rowbase = (b * a.dim + (active ? d : 0)) * L;

    // ---- B/C tile staging: element e -> (side, which, state, slot)
    constexpr int kTileElems = kSides * 2 * kRowLanes * kBlockTok;
    constexpr int kPerThread = (kTileElems + kThreads - 1) / kThreads;
    auto tile_src = [&](int e, int blk, float& v) {
        const int slot = e & 15, st_n = (e >> 4) & 15, which = (e >> 8) & 1, side = e >> 9;
        const int64_t t = static_cast<int64_t>(blk) * kBlockTok + slot;
        v = 0.f;
        if (t < L && st_n < a.dstate) {
            const T* src = which ? Cp : Bp;
            int64_t idx;
            if (MODE == kModeCross4) {
                idx = ((b * 4 + side) * a.dstate + st_n) * L + t;       // scan order
            } else {
                const int sorder = MODE == kModeVim ? side : order;
                const int64_t p = sorder == kRev ? L - 1 - t : t;
                idx = (b * a.dstate + st_n) * L + p;
            }
            v = ld(src, idx);
        }
    };
    float stage[kPerThread];
    auto stage_load = [&](int blk) {
#pragma unroll
        for (int r = 0; r < kPerThread; ++r) {
            const int e = tid + r * kThreads;
            stage[r] = 0.f;
            if (e < kTileElems) tile_src(e, blk, stage[r]);
        }
    };
    auto stage_store = [&](int buf) {
#pragma unroll
        for (int r = 0; r < kPerThread; ++r) {
            const int e = tid + r * kThreads;
            if (e < kTileElems) {
                const int slot = e & 15, st_n = (e >> 4) & 15, which = (e >> 8) & 1, side = e >> 9;
                tile[buf][side][which][st_n][slot] = stage[r];
            }
        }
    };

    // ---- per-lane token data for a block: token p of slot n (= lane in row)
    struct Tok { float u, dl, z; int64_t p; bool ok; };
    auto tok_load = [&](int blk) {
        Tok k;
        const int64_t t = static_cast<int64_t>(blk) * kBlockTok + n;
        k.ok = active && t < L;
        k.p = k.ok ? visit(order, t, L, a.H, a.W) : 0;
        k.u = k.ok ? ld(u, rowbase + k.p) : 0.f;
        k.dl = k.ok ? ld(dl, rowbase + k.p) : 0.f;
        k.z = (k.ok && z) ? ld(z, rowbase + k.p) : 0.f;
        return k;
    };

    stage_load(0);
    stage_store(0);
    Tok cur = tok_load(0);
    __syncthreads();

    float h = 0.f;
    for (int blk = 0; blk < a.nblk; ++blk) {
        const int buf = blk & 1;
        const bool more = blk + 1 < a.nblk;
        if (more) stage_load(blk + 1);
        Tok nxt{};
        if (more) nxt = tok_load(blk + 1);

        // delta and delta*u of this lane's token (zero for padding slots, so
        // they leave the state unchanged: exp(0) = 1, no input)
        float dlt = 0.f, du = 0.f;
        if (cur.ok) {
            const float x = cur.dl + bias;
            dlt = a.softplus ? softplus_f(x) : x;
            du = dlt * cur.u;
        }
        const int side = MODE == kMode1D ? 0 : dir;
        const float* Bt = &tile[buf][side][0][n][0];
        const float* Ct = &tile[buf][side][1][n][0];
        float c[16];
        Unroll<16>::run([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            const float e = __builtin_amdgcn_exp2f(row_bcast<i>(dlt) * A2);
            h = fmaf(e, h, row_bcast<i>(du) * Bt[i]);
            c[i] = Ct[i] * h;
        });
        const float yk = row_transpose_sum(c, lane) + Dk * cur.u;

        // ---- merge and store (lane n holds token slot n)
        if (MODE == kMode1D) {
            if (cur.ok) {
                float v = yk;
                if (z) v *= silu_f(cur.z);
                st(y, rowbase + cur.p, v);
            }
        } else if (MODE == kModeVim) {
            // This lane's scan step is t; the other direction visits the same
            // token at step L-1-t. The direction whose block finishes the
            // token first stores a partial sum; on a tie (both in this block
            // step) the forward row stores and the backward row finishes.
            const int64_t t_self = static_cast<int64_t>(blk) * kBlockTok + n;
            const int64_t blk_other = (L - 1 - t_self) / kBlockTok;
            const bool first = blk < blk_other || (blk == blk_other && dir == 0);
            if (cur.ok && first)
                __hip_atomic_store(&a.partial[rowbase + cur.p], yk, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            // block steps whose forward and backward blocks share tokens
            const int64_t b32 = static_cast<int64_t>(blk) * 2 * kBlockTok;
            if (L - 2 * kBlockTok + 1 <= b32 && b32 <= L - 1)
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
            if (cur.ok && !first) {
                const float other = __hip_atomic_load(&a.partial[rowbase + cur.p],
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                float v = yk + other;
                if (z) v *= silu_f(cur.z);
                st(y, rowbase + cur.p, v);
            }
        }

        if (more) stage_store(buf ^ 1);
        __syncthreads();
        if (more) cur = nxt;
    }
}

// ---------------------------------------------------------------- host side
thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

bool aligned(const void* p, size_t al) { return (reinterpret_cast<uintptr_t>(p) % al) == 0; }

struct Call {
    int mode;
    int64_t batch, dim, dstate, L;
    int H, W;
    int dtype;
    int reverse;
    const void *u, *delta, *z, *B, *C;
    const float *A, *Dskip, *dt_bias;
    int softplus;
    void* y;
    void* ws;
    size_t ws_bytes;
    void* stream;
};

int64_t ndirs(int mode) { return mode == kModeVim ? 2 : (mode == kModeCross4 ? 4 : 1); }

int validate(const Call& c) {
    if (c.dtype != VS_F32 && c.dtype != VS_BF16) return fail(VS_ERR_DTYPE, "unknown dtype");
    if (c.batch < 1 || c.dim < 1 || c.L < 1 || c.dstate < 1)
        return fail(VS_ERR_SHAPE, "batch, dim, dstate and the sequence length must be >= 1");
    if (c.dstate > VS_MAX_DSTATE)
        return fail(VS_ERR_UNSUPPORTED, "dstate above 16 is not supported");
    if (c.batch > 65535) return fail(VS_ERR_SHAPE, "batch above 65535 is not supported");
    if (c.L > (int64_t(1) << 30) || c.dim > (int64_t(1) << 30))
        return fail(VS_ERR_SHAPE, "sequence length or dim too large");
    const int64_t elems = c.batch * c.dim * c.L;
    if (elems > (int64_t(1) << 40)) return fail(VS_ERR_SHAPE, "problem too large");
    if (!c.u || !c.delta || !c.B || !c.C || !c.A || !c.y)
        return fail(VS_ERR_NULL, "u, delta, B, C, A and y must not be NULL");
    const size_t es = c.dtype == VS_BF16 ? 2 : 4;
    const void* acts[] = {c.u, c.delta, c.z, c.B, c.C, c.y};
    for (const void* p : acts)
        if (p && !aligned(p, es)) return fail(VS_ERR_ALIGN, "activation pointer misaligned");
    const void* fparams[] = {c.A, c.Dskip, c.dt_bias, c.ws};
    for (const void* p : fparams)
        if (p && !aligned(p, 4)) return fail(VS_ERR_ALIGN, "fp32 pointer misaligned");
    const int64_t nd = ndirs(c.mode);
    const size_t act = static_cast<size_t>(elems) * es;
    const size_t bc = static_cast<size_t>(c.batch * (c.mode == kModeCross4 ? 4 : 1) * c.dstate *
                                          c.L) * es;
    const size_t a_bytes = static_cast<size_t>(nd * c.dim * c.dstate) * 4;
    const size_t p_bytes = static_cast<size_t>(nd * c.dim) * 4;
    const void* ins[] = {c.u, c.delta, c.z, c.B, c.C, c.A, c.Dskip, c.dt_bias};
    const size_t in_bytes[] = {act, act, act, bc, bc, a_bytes, p_bytes, p_bytes};
    for (int i = 0; i < 8; ++i)
        if (overlaps(c.y, act, ins[i], in_bytes[i]))
            return fail(VS_ERR_ALIAS, "y overlaps an input");
    const size_t need = vs_workspace_bytes(
        c.mode == kModeVim ? VS_OP_VIM_BIDIR : (c.mode == kModeCross4 ? VS_OP_CROSS4 : VS_OP_1D),
        c.batch, c.dim, c.L, c.dtype);
    if (need > 0) {
        if (!c.ws || c.ws_bytes < need)
            return fail(VS_ERR_WORKSPACE, "workspace missing or smaller than vs_workspace_bytes()");
        if (overlaps(c.y, act, c.ws, need)) return fail(VS_ERR_ALIAS, "y overlaps the workspace");
        for (int i = 0; i < 8; ++i)
            if (overlaps(c.ws, need, ins[i], in_bytes[i]))
                return fail(VS_ERR_ALIAS, "workspace overlaps an input");
    }
    if (c.mode == kModeCross4 && (c.H < 1 || c.W < 1 || int64_t(c.H) * c.W != c.L))
        return fail(VS_ERR_SHAPE, "H and W must be >= 1 with H*W = L");
    return VS_OK;
}

template <typename T, int MODE>
int launch_t(const Call& c) {
    ScanArgs a;
    a.u = c.u; a.delta = c.delta; a.z = c.z; a.B = c.B; a.C = c.C;
    a.A = c.A; a.Dskip = c.Dskip; a.dt_bias = c.dt_bias; a.y = c.y;
    a.partial = c.dtype == VS_F32 ? static_cast<float*>(c.y) : static_cast<float*>(c.ws);
    a.dim = c.dim; a.L = c.L; a.H = c.H; a.W = c.W;
    a.dstate = static_cast<int>(c.dstate);
    a.softplus = c.softplus ? 1 : 0;
    a.reverse = c.reverse ? 1 : 0;
    a.nblk = static_cast<int>((c.L + kBlockTok - 1) / kBlockTok);
    constexpr int kChPerWg = MODE == kModeVim ? 8 : (MODE == kModeCross4 ? 4 : 16);
    dim3 grid(static_cast<unsigned>((c.dim + kChPerWg - 1) / kChPerWg),
              static_cast<unsigned>(c.batch));
    hipLaunchKernelGGL((rowscan_kernel<T, MODE>), grid, dim3(kThreads), 0,
                       static_cast<hipStream_t>(c.stream), a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(VS_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return VS_OK;
}

int run(const Call& c) {
    g_last_error.clear();
    int rc = validate(c);
    if (rc != VS_OK) return rc;
    const bool bf = c.dtype == VS_BF16;
    switch (c.mode) {
    case kMode1D: return bf ? launch_t<uint16_t, kMode1D>(c) : launch_t<float, kMode1D>(c);
    case kModeVim: return bf ? launch_t<uint16_t, kModeVim>(c) : launch_t<float, kModeVim>(c);
    default: return fail(VS_ERR_UNSUPPORTED, "cross-scan is not built yet");
    }
}

}  // namespace

// ---------------------------------------------------------------- C ABI
extern "C" {

size_t vs_workspace_bytes(int op, int64_t batch, int64_t dim, int64_t seqlen, int dtype) {
    if (batch < 1 || dim < 1 || seqlen < 1) return 0;
    if (dtype != VS_BF16) return 0;            // fp32 y holds the partial sums
    if (op == VS_OP_VIM_BIDIR || op == VS_OP_CROSS4)
        return static_cast<size_t>(batch * dim * seqlen) * sizeof(float);
    return 0;
}

int vim_scan_bidir(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                   const void* u, const void* delta, const void* z, const void* B,
                   const void* C, const float* A, const float* Dskip, const float* dt_bias,
                   int delta_softplus, void* y, void* workspace, size_t workspace_bytes,
                   void* stream) {
    Call c{kModeVim, batch, dim, dstate, seqlen, 0, 0, dtype, 0, u, delta, z, B, C,
           A, Dskip, dt_bias, delta_softplus, y, workspace, workspace_bytes, stream};
    return run(c);
}

int vmamba_cross_scan4(int64_t batch, int64_t dim, int64_t dstate, int64_t H, int64_t W,
                       int dtype, const void* u, const void* delta, const void* z,
                       const void* B, const void* C, const float* A, const float* Dskip,
                       const float* dt_bias, int delta_softplus, void* y, void* workspace,
                       size_t workspace_bytes, void* stream) {
    if (H < 1 || W < 1 || H > (int64_t(1) << 20) || W > (int64_t(1) << 20)) {
        g_last_error = "H and W must be in 1..2^20";
        return VS_ERR_SHAPE;
    }
    Call c{kModeCross4, batch, dim, dstate, H * W, static_cast<int>(H), static_cast<int>(W),
           dtype, 0, u, delta, z, B, C, A, Dskip, dt_bias, delta_softplus, y, workspace,
           workspace_bytes, stream};
    return run(c);
}

int s6_scan_1d(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
               int reverse, const void* u, const void* delta, const void* z, const void* B,
               const void* C, const float* A, const float* Dskip, const float* dt_bias,
               int delta_softplus, void* y, void* stream) {
    Call c{kMode1D, batch, dim, dstate, seqlen, 0, 0, dtype, reverse, u, delta, z, B, C,
           A, Dskip, dt_bias, delta_softplus, y, nullptr, 0, stream};
    return run(c);
}

const char* vs_strerror(int status) {
    switch (status) {
    case VS_OK: return "VS_OK";
    case VS_ERR_NULL: return "VS_ERR_NULL";
    case VS_ERR_SHAPE: return "VS_ERR_SHAPE";
    case VS_ERR_DTYPE: return "VS_ERR_DTYPE";
    case VS_ERR_ALIGN: return "VS_ERR_ALIGN";
    case VS_ERR_ALIAS: return "VS_ERR_ALIAS";
    case VS_ERR_UNSUPPORTED: return "VS_ERR_UNSUPPORTED";
    case VS_ERR_HIP: return "VS_ERR_HIP";
    case VS_ERR_WORKSPACE: return "VS_ERR_WORKSPACE";
    default: return "VS_ERR_UNKNOWN";
    }
}

const char* vs_last_error(void) { return g_last_error.c_str(); }

int vs_abi_version(void) { return VS_ABI_VERSION; }

}  // extern "C"
