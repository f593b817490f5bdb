// host.cpp -- the host-side layer of libvimscan.so: argument validation,
// workspace layout and the error record. Plain C++ with no HIP: every check
// here runs before the kernel translation units touch the HIP runtime, and
// the file builds on its own (the CPU tests build it under the address and
// undefined-behaviour sanitizers).
#include <cstdint>
#include <string>

#include "vs_internal.h"

namespace vs {

namespace {
thread_local std::string g_last_error;
}

int fail(int code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

void clear_error() { g_last_error.clear(); }

const char* last_error() { return g_last_error.c_str(); }

bool product_below(int64_t a, int64_t b, int64_t c, int64_t limit) {
    if (a < 1 || b < 1 || c < 1 || limit < 1) return false;
    if (a >= limit || b >= limit || c >= limit) return false;
    if (a > (limit - 1) / b) return false;
    const int64_t ab = a * b;            // < limit
    return ab <= (limit - 1) / c;        // then ab * c < limit
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    // a0 < b0 + nb and b0 < a0 + na, without wrapping past the address space
    return (a0 < b0 || a0 - b0 < nb) && (b0 < a0 || b0 - a0 < na);
}

bool aligned(const void* p, size_t al) { return (reinterpret_cast<uintptr_t>(p) % al) == 0; }

int64_t ndirs(int mode) { return mode == kModeVim ? 2 : (mode == kModeCross4 ? 4 : 1); }

size_t scan_ws_bytes(int op, int64_t batch, int64_t dim, int64_t seqlen, int dtype) {
    if (batch < 1 || dim < 1 || seqlen < 1) return 0;
    if (dtype != VS_F32 && dtype != VS_BF16) return 0;
    // every entry point refuses 2^30 elements or more; the products below
    // are formed only for sizes under that
    if (!product_below(batch, dim, seqlen, kMaxElems)) return 0;
    if (op == VS_OP_VIM_GRAD) {
        size_t offs[6];
        return grad_ws_bytes(batch, dim, seqlen, offs);
    }
    if (op == VS_OP_VIM_SAVED) {
        size_t offs[2];
        return grad_saved_bytes(batch, dim, seqlen, offs);
    }
    if (op == VS_OP_VIM_GRAD_SAVED) {
        size_t offs[4];
        return grad_rest_bytes(batch, dim, seqlen, offs);
    }
    if (op != VS_OP_VIM_BIDIR && op != VS_OP_CROSS4 && op != VS_OP_1D) return 0;
    // fp32 merge buffers of batch*dim*seqlen floats: Vim needs one, the
    // cross-scan two; an fp32 y serves as the first. The cross-scan also
    // keeps column-major copies of u and delta (input dtype) when the grid
    // is too large to stage in LDS.
    const int64_t elems = batch * dim * seqlen;
    const int64_t bufs = (op == VS_OP_VIM_BIDIR ? 1 : (op == VS_OP_CROSS4 ? 2 : 0)) -
                         (dtype == VS_F32 ? 1 : 0);
    const int64_t copies = (op == VS_OP_CROSS4 && !cross4_grid_in_lds(seqlen, dtype)) ? 2 : 0;
    const int64_t es = dtype == VS_BF16 ? 2 : 4;
    if (bufs <= 0 && copies == 0) return 0;
    return static_cast<size_t>(elems * (4 * (bufs > 0 ? bufs : 0) + es * copies));
}

namespace {

int validate(const Call& c) {
    if (c.dtype != VS_F32 && c.dtype != VS_BF16) return fail(VS_ERR_DTYPE, "unknown dtype");
    if (c.batch < 1 || c.dim < 1 || c.L < 1 || c.dstate < 1)
        return fail(VS_ERR_SHAPE, "batch, dim, dstate and the sequence length must be >= 1");
    if (c.dstate > VS_MAX_DSTATE)
        return fail(VS_ERR_UNSUPPORTED, "dstate above 16 is not supported");
    if (c.batch > 65535) return fail(VS_ERR_SHAPE, "batch above 65535 is not supported");
    if (c.L > kMaxElems || c.dim > kMaxElems)
        return fail(VS_ERR_SHAPE, "sequence length or dim too large");
    if (c.chunks < 0) return fail(VS_ERR_SHAPE, "the chunk count must be >= 0");
    if (c.chunks > 1 && (c.mode != kModeVim || c.conv || c.zoh || c.per_dir))
        return fail(VS_ERR_UNSUPPORTED, "chunks: the plain Vim scan only (no ZOH)");
    if (c.saved_fwd && c.zoh)
        return fail(VS_ERR_UNSUPPORTED, "the saving forward takes VS_FLAG_SOFTPLUS only (delta B form)");
    if (c.saved_fwd && c.L > kGradMaxL)
        return fail(VS_ERR_UNSUPPORTED, "the saving forward supports sequences of up to 2^26 tokens");
    // kernels address every tensor with 32-bit byte offsets (fp32 partial
    // sums included), so each tensor must stay below 4 GiB. Every factor is
    // bounded above by now, and the products are formed only once they are
    // known to stay below 2^30.
    const int64_t copies = c.per_dir ? 2 : 1;     // direction copies of u, delta, B and C
    if (!product_below(c.batch, c.dim, c.L, kMaxElems) ||
        !product_below(c.batch, 4 * c.dstate, c.L, kMaxElems) ||
        !product_below(copies * c.batch, c.dim, c.L, kMaxElems))
        return fail(VS_ERR_UNSUPPORTED, "tensors of 2^30 elements or more are not supported");
    const int64_t elems = c.batch * c.dim * c.L;
    if (c.conv && !c.conv_w) return fail(VS_ERR_NULL, "conv_w must not be NULL");
    if (!c.u || !c.delta || !c.B || !c.C || !c.A || !c.y)
        return fail(VS_ERR_NULL, "u, delta, B, C, A and y must not be NULL");
    const size_t es = c.dtype == VS_BF16 ? 2 : 4;
    const void* acts[] = {c.u, c.delta, c.z, c.B, c.C, c.y};
    for (const void* p : acts)
        if (p && !aligned(p, es)) return fail(VS_ERR_ALIGN, "activation pointer misaligned");
    const void* fparams[] = {c.A, c.Dskip, c.dt_bias, c.ws, c.conv_w, c.conv_b};
    for (const void* p : fparams)
        if (p && !aligned(p, 4)) return fail(VS_ERR_ALIGN, "fp32 pointer misaligned");
    const int64_t nd = ndirs(c.mode);
    const size_t act = static_cast<size_t>(elems) * es;
    const size_t bc = static_cast<size_t>(c.batch * (c.mode == kModeCross4 ? 4 : copies) *
                                          c.dstate * c.L) * es;
    const size_t act_in = act * static_cast<size_t>(copies);
    const size_t a_bytes = static_cast<size_t>(nd * c.dim * c.dstate) * 4;
    const size_t p_bytes = static_cast<size_t>(nd * c.dim) * 4;
    const void* ins[] = {c.u, c.delta, c.z, c.B, c.C, c.A, c.Dskip, c.dt_bias, c.conv_w, c.conv_b};
    const size_t in_bytes[] = {act_in, act_in, act, bc, bc, a_bytes, p_bytes, p_bytes, 3 * p_bytes,
                               p_bytes};
    constexpr int kIns = 10;
    for (int i = 0; i < kIns; ++i)
        if (overlaps(c.y, act, ins[i], in_bytes[i]))
            return fail(VS_ERR_ALIAS, "y overlaps an input");
    const size_t need = scan_ws_bytes(
        c.saved_fwd ? VS_OP_VIM_SAVED
                    : (c.mode == kModeVim ? VS_OP_VIM_BIDIR : (c.mode == kModeCross4 ? VS_OP_CROSS4 : VS_OP_1D)),
        c.batch, c.dim, c.L, c.dtype);
    if (need > 0 && c.ws_internal) {
        // the library's own buffer: no overlap with the caller's memory is
        // possible, only its capacity can fall short
        if (c.ws_bytes < need)
            return fail(VS_ERR_UNSUPPORTED, "batch*dim*seqlen above the no-allocation maximum "
                                            "(VS_NOALLOC_MAX_ELEMS for bf16)");
    } else if (need > 0) {
        if (!c.ws || c.ws_bytes < need)
            return fail(VS_ERR_WORKSPACE, c.saved_fwd ? "saved-state buffer missing or smaller than "
                                                        "vs_workspace_bytes(VS_OP_VIM_SAVED)"
                                                      : "workspace missing or smaller than vs_workspace_bytes()");
        if (overlaps(c.y, act, c.ws, need)) return fail(VS_ERR_ALIAS, "y overlaps the workspace");
        for (int i = 0; i < kIns; ++i)
            if (overlaps(c.ws, need, ins[i], in_bytes[i]))
                return fail(VS_ERR_ALIAS, "workspace overlaps an input");
    }
    if (c.mode == kModeCross4 && (c.H < 1 || c.W < 1 || int64_t(c.H) * c.W != c.L))
        return fail(VS_ERR_SHAPE, "H and W must be >= 1 with H*W = L");
    return VS_OK;
}

}  // namespace

int prepare(Call& c) {
    clear_error();
    // the delta_softplus argument is a flags word: VS_FLAG_SOFTPLUS, VS_FLAG_ZOH
    if (c.softplus & ~(VS_FLAG_SOFTPLUS | VS_FLAG_ZOH))
        return fail(VS_ERR_UNSUPPORTED, "unknown flag bits");
    c.zoh = (c.softplus & VS_FLAG_ZOH) != 0;
    c.softplus &= VS_FLAG_SOFTPLUS;
    return validate(c);
}

// Channels per gradient workgroup. With 24 (768 threads, one workgroup per
// CU at 3 waves per SIMD) the workgroups write a third of the dB/dC chunks
// that 8 channels (256 threads) write; 24 is used when it still gives every
// one of the 256 CUs a workgroup.
int grad_channels(int64_t batch, int64_t dim) {
    return batch * ((dim + 23) / 24) >= kNumCUs ? 24 : 8;
}

// The gradient's buffers, each region 256-byte aligned. Sizes must have
// passed the 2^30-element checks.
namespace {
size_t al256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
}

// saved part: [s: fp32 E, the merged ungated forward output][checkpoints:
// fp32 [batch][dim][2][nblk][16], the state at every block start]
size_t grad_saved_bytes(int64_t batch, int64_t dim, int64_t L, size_t offs[2]) {
    const size_t elems = static_cast<size_t>(batch * dim * L);
    const size_t nblk = static_cast<size_t>((L + kBlockTok - 1) / kBlockTok);
    const size_t ck = static_cast<size_t>(batch * dim) * 2 * nblk * kRowLanes;
    offs[0] = 0;
    offs[1] = al256(4 * elems);
    return offs[1] + al256(4 * ck);
}

// rest: [du partials: fp32 E][ddelta partials: fp32 E][dB/dC chunks]
// [per batch row: dA [2][dim][dstate], dD [2][dim], ddt_bias [2][dim], sized
// for the largest dstate]
size_t grad_rest_bytes(int64_t batch, int64_t dim, int64_t L, size_t offs[4]) {
    const size_t elems = static_cast<size_t>(batch * dim * L);
    const size_t nblk = static_cast<size_t>((L + kBlockTok - 1) / kBlockTok);
    const int ch = grad_channels(batch, dim);
    const size_t groups = static_cast<size_t>((dim + ch - 1) / ch);
    const size_t chunks = static_cast<size_t>(batch) * groups * nblk * kBcChunk;
    size_t off = 0;
    offs[0] = off; off += al256(4 * elems);
    offs[1] = off; off += al256(4 * elems);
    offs[2] = off; off += al256(4 * chunks);
    offs[3] = off; off += al256(4 * static_cast<size_t>(batch * 2 * dim * (VS_MAX_DSTATE + 2)));
    return off;
}

// the whole gradient workspace: the saved part, then the rest
size_t grad_ws_bytes(int64_t batch, int64_t dim, int64_t L, size_t offs[6]) {
    size_t so[2], ro[4];
    const size_t saved = grad_saved_bytes(batch, dim, L, so);
    const size_t rest = grad_rest_bytes(batch, dim, L, ro);
    offs[0] = so[0];
    offs[1] = so[1];
    for (int i = 0; i < 4; ++i) offs[2 + i] = saved + ro[i];
    return saved + rest;
}

int validate_grad(const GradCall& g) {
    if (g.dtype != VS_F32 && g.dtype != VS_BF16) return fail(VS_ERR_DTYPE, "unknown dtype");
    if (g.softplus & ~VS_FLAG_SOFTPLUS)
        return fail(VS_ERR_UNSUPPORTED, "the gradient takes VS_FLAG_SOFTPLUS only (delta B form)");
    if (g.batch < 1 || g.dim < 1 || g.L < 1 || g.dstate < 1)
        return fail(VS_ERR_SHAPE, "batch, dim, dstate and the sequence length must be >= 1");
    if (g.dstate > VS_MAX_DSTATE)
        return fail(VS_ERR_UNSUPPORTED, "dstate above 16 is not supported");
    if (g.batch > 65535) return fail(VS_ERR_SHAPE, "batch above 65535 is not supported");
    if (g.L > kMaxElems || g.dim > kMaxElems)
        return fail(VS_ERR_SHAPE, "sequence length or dim too large");
    if (!product_below(g.batch, g.dim, g.L, kMaxElems) || !product_below(g.batch, g.dstate, g.L, kMaxElems))
        return fail(VS_ERR_UNSUPPORTED, "tensors of 2^30 elements or more are not supported");
    const int64_t elems = g.batch * g.dim * g.L;
    if (g.L > kGradMaxL) return fail(VS_ERR_UNSUPPORTED, "the gradient supports sequences of up to 2^26 tokens");
    if (!g.u || !g.delta || !g.B || !g.C || !g.A || !g.dy)
        return fail(VS_ERR_NULL, "u, delta, B, C, A and dy must not be NULL");
    if (!g.du || !g.ddelta || !g.dB || !g.dC || !g.dA || !g.dD || !g.dbias)
        return fail(VS_ERR_NULL, "every gradient output must be given");
    if (g.z && !g.dz) return fail(VS_ERR_NULL, "dz must not be NULL when z is given");
    const size_t es = g.dtype == VS_BF16 ? 2 : 4;
    const void* acts[] = {g.u, g.delta, g.z, g.B, g.C, g.dy, g.du, g.ddelta, g.dz};
    for (const void* p : acts)
        if (p && !aligned(p, es)) return fail(VS_ERR_ALIGN, "activation pointer misaligned");
    const void* fps[] = {g.A, g.Dskip, g.dt_bias, g.dB, g.dC, g.dA, g.dD, g.dbias, g.ws, g.saved};
    for (const void* p : fps)
        if (p && !aligned(p, 4)) return fail(VS_ERR_ALIGN, "fp32 pointer misaligned");
    size_t offs[6];
    const size_t need = g.saved ? grad_rest_bytes(g.batch, g.dim, g.L, offs)
                                : grad_ws_bytes(g.batch, g.dim, g.L, offs);
    if (!g.ws || g.ws_bytes < need)
        return fail(VS_ERR_WORKSPACE, "workspace missing or smaller than vs_workspace_bytes()");
    const size_t saved_need = grad_saved_bytes(g.batch, g.dim, g.L, offs);
    if (g.saved && g.saved_bytes < saved_need)
        return fail(VS_ERR_WORKSPACE, "saved-state buffer smaller than vs_workspace_bytes(VS_OP_VIM_SAVED)");
    // no output (nor the workspace) may overlap an input or another output
    const size_t act = static_cast<size_t>(elems) * es;
    const size_t bc_in = static_cast<size_t>(g.batch * g.dstate * g.L) * es;
    const size_t bcf = static_cast<size_t>(g.batch * g.dstate * g.L) * 4;
    const size_t pa = static_cast<size_t>(2 * g.dim * g.dstate) * 4;
    const size_t pd = static_cast<size_t>(2 * g.dim) * 4;
    const void* ins[] = {g.u, g.delta, g.z, g.B, g.C, g.A, g.Dskip, g.dt_bias, g.dy, g.saved};
    const size_t in_b[] = {act, act, act, bc_in, bc_in, pa, pd, pd, act, g.saved ? saved_need : 0};
    const void* outs[] = {g.du, g.ddelta, g.dz, g.dB, g.dC, g.dA, g.dD, g.dbias, g.ws};
    const size_t out_b[] = {act, act, act, bcf, bcf, pa, pd, pd, need};
    for (int i = 0; i < 9; ++i) {
        for (int j = 0; j < 10; ++j)
            if (overlaps(outs[i], out_b[i], ins[j], in_b[j]))
                return fail(VS_ERR_ALIAS, "a gradient output or the workspace overlaps an input");
        for (int j = i + 1; j < 9; ++j)
            if (overlaps(outs[i], out_b[i], outs[j], out_b[j]))
                return fail(VS_ERR_ALIAS, "gradient outputs overlap each other or the workspace");
    }
    return VS_OK;
}

// ---- the linear maps
namespace {

constexpr int64_t kProjMax = int64_t(1) << 31;

int proj_dtype(int dtype) {
    if (dtype == VS_BF16) return VS_OK;
    return dtype == VS_F32 ? fail(VS_ERR_UNSUPPORTED, "the projections take bf16 only")
                           : fail(VS_ERR_DTYPE, "unknown dtype");
}

int check_sizes(int64_t batch, int64_t M, int64_t K, int64_t L) {
    if (batch < 1 || M < 1 || K < 1 || L < 1)
        return fail(VS_ERR_SHAPE, "batch, feature counts and the sequence length must be >= 1");
    if (batch > 65535) return fail(VS_ERR_SHAPE, "batch above 65535 is not supported");
    if (L >= (int64_t(1) << 30) || !product_below(M, K, 1, kProjMax) ||
        !product_below(batch, K, L, kProjMax) || !product_below(batch, M, L, kProjMax))
        return fail(VS_ERR_UNSUPPORTED, "tensors of 2^31 elements or more are not supported");
    return VS_OK;
}

}  // namespace

int validate_x_proj(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                    const void* u, const void* W, const void* B, const void* C, const float* dt) {
    clear_error();
    int rc = proj_dtype(dtype);
    if (rc != VS_OK) return rc;
    if (dstate < 1 || dstate > VS_MAX_DSTATE)
        return fail(dstate < 1 ? VS_ERR_SHAPE : VS_ERR_UNSUPPORTED, "dstate must be in 1..16");
    const int64_t M = 2 * dstate + 1;
    rc = check_sizes(batch, M, dim, seqlen);
    if (rc != VS_OK) return rc;
    if (!u || !W || !B || !C || !dt) return fail(VS_ERR_NULL, "u, W, B, C and dt must not be NULL");
    if (!aligned(u, 2) || !aligned(W, 2) || !aligned(B, 2) || !aligned(C, 2) || !aligned(dt, 4))
        return fail(VS_ERR_ALIGN, "pointer misaligned");
    const size_t nu = static_cast<size_t>(batch * dim * seqlen) * 2, nw = static_cast<size_t>(M * dim) * 2;
    const size_t nbc = static_cast<size_t>(batch * dstate * seqlen) * 2;
    const size_t ndt = static_cast<size_t>(batch * seqlen) * 4;
    const void* outs[] = {B, C, dt};
    const size_t out_b[] = {nbc, nbc, ndt};
    for (int i = 0; i < 3; ++i) {
        if (overlaps(outs[i], out_b[i], u, nu) || overlaps(outs[i], out_b[i], W, nw))
            return fail(VS_ERR_ALIAS, "an output overlaps an input");
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], out_b[i], outs[j], out_b[j]))
                return fail(VS_ERR_ALIAS, "outputs overlap each other");
    }
    return VS_OK;
}

int validate_dt_proj(int64_t batch, int64_t dim, int64_t seqlen, int dtype, const float* dt,
                     const float* w, const void* delta) {
    clear_error();
    int rc = proj_dtype(dtype);
    if (rc != VS_OK) return rc;
    rc = check_sizes(batch, dim, 1, seqlen);
    if (rc != VS_OK) return rc;
    if (dim > 65535) return fail(VS_ERR_UNSUPPORTED, "dim above 65535 is not supported");
    if (!dt || !w || !delta) return fail(VS_ERR_NULL, "dt, w and delta must not be NULL");
    if (!aligned(dt, 4) || !aligned(w, 4) || !aligned(delta, 2)) return fail(VS_ERR_ALIGN, "pointer misaligned");
    const size_t nd = static_cast<size_t>(batch * dim * seqlen) * 2;
    if (overlaps(delta, nd, dt, static_cast<size_t>(batch * seqlen) * 4) ||
        overlaps(delta, nd, w, static_cast<size_t>(dim) * 4))
        return fail(VS_ERR_ALIAS, "delta overlaps an input");
    return VS_OK;
}

int validate_out_proj(int64_t batch, int64_t dim_in, int64_t dim_out, int64_t seqlen, int dtype,
                      const void* y, const void* W, const float* bias, const void* residual,
                      const void* out) {
    clear_error();
    int rc = proj_dtype(dtype);
    if (rc != VS_OK) return rc;
    rc = check_sizes(batch, dim_out, dim_in, seqlen);
    if (rc != VS_OK) return rc;
    if (!y || !W || !out) return fail(VS_ERR_NULL, "y, W and out must not be NULL");
    if (!aligned(y, 2) || !aligned(W, 2) || !aligned(out, 2) || !aligned(residual, 2) || !aligned(bias, 4))
        return fail(VS_ERR_ALIGN, "pointer misaligned");
    const size_t no = static_cast<size_t>(batch * dim_out * seqlen) * 2;
    if (overlaps(out, no, y, static_cast<size_t>(batch * dim_in * seqlen) * 2) ||
        overlaps(out, no, W, static_cast<size_t>(dim_out * dim_in) * 2) ||
        overlaps(out, no, bias, static_cast<size_t>(dim_out) * 4))
        return fail(VS_ERR_ALIAS, "out overlaps an input");
    // out may be the residual itself (each element is read before it is
    // written, by the same thread); any other overlap is refused
    if (residual != out && overlaps(out, no, residual, no))
        return fail(VS_ERR_ALIAS, "out partly overlaps the residual");
    return VS_OK;
}

}  // namespace vs

// ---------------------------------------------------------------- C ABI
extern "C" {

size_t vs_workspace_bytes(int op, int64_t batch, int64_t dim, int64_t seqlen, int dtype) {
    return vs::scan_ws_bytes(op, batch, dim, seqlen, dtype);
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

const char* vs_last_error(void) { return vs::last_error(); }

int vs_abi_version(void) { return VS_ABI_VERSION; }

}  // extern "C"
