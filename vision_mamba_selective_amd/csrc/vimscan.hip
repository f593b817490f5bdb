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
//     batch*dim*ndir*16 lanes: enough waves to fill 256 CUs at batch 2-8 for
//     most shapes. Grids that leave SIMDs idle split the sequence into
//     chunks joined by the associative carry combine (the CHUNK form), at
//     the cost of a first pass over the other chunks' tokens.
//   * Tokens are processed in blocks of 16. Lane j of a row loads token j of
//     the block (coalesced within the row), computes its delta = softplus(.)
//     and delta*u once, and the row broadcasts them to every state lane with
//     DPP row_newbcast, so no state lane repeats the softplus.
//   * B and C rows of a block are shared by every channel of a batch: the
//     workgroup stages them once per block in LDS (converted to fp32), and each
//     state lane reads its own 16-token window.
//   * The read-out sum over states (y = C . h) is a 16-lane transpose
//     reduction inside the row after each block: lane j ends with token j.
//   * Reverse orders are index arithmetic on the token address; nothing is
//     flipped in memory. The VMamba column-major pair reads u and delta by
//     their column-major index: from an LDS copy that the workgroup writes
//     in that order when the grid fits (the GLDS form), otherwise from
//     column-major copies that a transpose pre-pass writes to the workspace
//     (strided reads of the row-major grid measured 2.5x slower).
//   * Directions that visit a token at different times meet through an fp32
//     partial sum (a workspace, or y itself when y is fp32): the first
//     direction to finish a token stores its contribution, the last one adds
//     it, applies the gate and writes y once.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>

#include "vimscan.h"
#include "vs_internal.h"

namespace {

constexpr int kWaveLanes = 64;
using vs::kRowLanes;                // one recurrence per DPP row
using vs::kBlockTok;                // tokens per block step
constexpr int kThreads = 256;       // 4 waves per workgroup
constexpr int kTilePad = 20;        // LDS row stride (floats) of a 16-token tile
constexpr int kTokAhead = 3;        // blocks the forward scan's token loads run ahead
constexpr int kTr = 32;             // grid transpose tile edge
constexpr int kTrPad = kTr + 1;

using vs::kMode1D;
using vs::kModeVim;
using vs::kModeCross4;

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
    float* partial2;    // cross-scan: the column-major pair's partial sums
    const void* uT;     // cross-scan: u and delta transposed to column-major
    const void* deltaT;
    float* ckpt;            // gradient recompute: state at each block start
    const float* conv_w;    // Vim front end: depthwise taps [2][dim][3] (u holds x)
    const float* conv_b;    // and biases [2][dim] (NULL: 0)
    // Vim with per-direction inputs: the backward rows read u and delta this
    // many elements past the forward rows' (0: shared), and B, C are
    // [batch][2][dstate][L] in token order when bc_per_dir is set
    uint32_t dir_off;
    int bc_per_dir;
    int64_t dim;
    int64_t L;
    int H;
    int W;
    int dstate;
    int softplus;
    int reverse;        // 1-D mode only
    int nblk;           // ceil(L / 16)
    int nchunk;         // chunked Vim scan: chunks per sequence (grid.y = batch * nchunk)
};

// The kernels' per-block steps are lambdas over register arrays (token
// sets, tiles' raw words); one left out of line would put those arrays in
// scratch memory.
#define VS_INLINE __attribute__((always_inline))

// ---------------------------------------------------------------- dtype I/O
__device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
// Raw loads keep the loaded bits untouched so that the conversion (and the
// wait for the load) happens where the value is used, not where it is loaded.
__device__ __forceinline__ uint32_t ld_raw(const float* p, int64_t i) { return __float_as_uint(p[i]); }
__device__ __forceinline__ uint32_t ld_raw(const uint16_t* p, int64_t i) { return p[i]; }
template <typename T>
__device__ __forceinline__ float from_raw(uint32_t r) {
    if constexpr (sizeof(T) == 2) return __uint_as_float(r << 16);
    else return __uint_as_float(r);
}
__device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) {
    p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

// ------------------------------------------------------------- lane moves
// DPP move whose result feeds a VALU op; the compiler folds it into the
// consumer (v_mul_f32_dpp etc.) when both operands are VGPRs.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
// value of lane I of this 16-lane row, in every lane of the row (row_newbcast)
template <int I>
__device__ __forceinline__ float row_bcast(float v) { return dpp<0x150 + I>(v); }
// acc + row_bcast<I>(v) * w as one v_fmac_f32_dpp. The compiler does not fold
// a DPP move into fmac (whose accumulator is tied to its result), so the
// instruction is written out, and the compiler does not see its DPP read: a
// DPP source needs two wait states after its VALU write. With FIRST the asm
// opens with s_nop 1, for the first of a chain of calls that read one source;
// the later calls of the chain read the same value, written before the
// first. tests/test_dpp_hazards.py checks the rule on every path of the
// built code object.
template <int I, bool FIRST>
__device__ __forceinline__ float row_bcast_fmac(float acc, float v, float w) {
    static_assert(I >= 0 && I < 16, "a lane of the row");
    if constexpr (FIRST)
        asm("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
            : "+v"(acc) : "v"(v), "v"(w), "i"(I));
    else
        asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
            : "+v"(acc) : "v"(v), "v"(w), "i"(I));
    return acc;
}

// Transpose-reduce across the 16 lanes of a row: lane n holds c[i] = its
// state's share of token i's read-out; on return lane j holds the sum over
// the row's lanes of c[j]. Each halving stage pairs lane j with lane j^m. The
// two cross-bank stages (m = 8, 4) write the kept half of each bank (4-lane
// group) with bank-masked DPP adds, 2 per pair, in one asm block: its
// leading s_nop gives the two wait states a DPP read needs after the VALU
// write of its source, and inside the block every DPP source was written at
// least 7 instructions earlier; the trailing s_nop covers the DPP reads that
// follow the block. The in-bank stages (m = 2, 1) add both halves and select.
#define VS_ADD8(T, C, K) \
    "v_add_f32_dpp %[" #T "], %[" #C "], %[" #C "] row_ror:8 row_mask:0xf bank_mask:" K "\n\t"
#define VS_ADD4(V, T, R, K) \
    "v_add_f32_dpp %[" #V "], %[" #T "], %[" #T "] " R " row_mask:0xf bank_mask:" K "\n\t"
__device__ __forceinline__ float row_transpose_sum(const float (&c)[16], int lane) {
    float t0, t1, t2, t3, t4, t5, t6, t7, v0, v1, v2, v3;
    asm("s_nop 1\n\t"
        VS_ADD8(t0, c0, "0x3") VS_ADD8(t0, c8, "0xc")
        VS_ADD8(t1, c1, "0x3") VS_ADD8(t1, c9, "0xc")
        VS_ADD8(t2, c2, "0x3") VS_ADD8(t2, c10, "0xc")
        VS_ADD8(t3, c3, "0x3") VS_ADD8(t3, c11, "0xc")
        VS_ADD8(t4, c4, "0x3") VS_ADD8(t4, c12, "0xc")
        VS_ADD8(t5, c5, "0x3") VS_ADD8(t5, c13, "0xc")
        VS_ADD8(t6, c6, "0x3") VS_ADD8(t6, c14, "0xc")
        VS_ADD8(t7, c7, "0x3") VS_ADD8(t7, c15, "0xc")
        VS_ADD4(v0, t0, "row_ror:12", "0x5") VS_ADD4(v0, t4, "row_ror:4", "0xa")
        VS_ADD4(v1, t1, "row_ror:12", "0x5") VS_ADD4(v1, t5, "row_ror:4", "0xa")
        VS_ADD4(v2, t2, "row_ror:12", "0x5") VS_ADD4(v2, t6, "row_ror:4", "0xa")
        VS_ADD4(v3, t3, "row_ror:12", "0x5") VS_ADD4(v3, t7, "row_ror:4", "0xa")
        "s_nop 1"
        : [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2), [t3] "=&v"(t3), [t4] "=&v"(t4),
          [t5] "=&v"(t5), [t6] "=&v"(t6), [t7] "=&v"(t7), [v0] "=&v"(v0), [v1] "=&v"(v1),
          [v2] "=&v"(v2), [v3] "=&v"(v3)
        : [c0] "v"(c[0]), [c1] "v"(c[1]), [c2] "v"(c[2]), [c3] "v"(c[3]), [c4] "v"(c[4]),
          [c5] "v"(c[5]), [c6] "v"(c[6]), [c7] "v"(c[7]), [c8] "v"(c[8]), [c9] "v"(c[9]),
          [c10] "v"(c[10]), [c11] "v"(c[11]), [c12] "v"(c[12]), [c13] "v"(c[13]),
          [c14] "v"(c[14]), [c15] "v"(c[15]));
    const bool b1 = (lane & 2) != 0, b0 = (lane & 1) != 0;
    const float s0 = v0 + dpp<0x4e>(v0), s2 = v2 + dpp<0x4e>(v2);   // quad_perm [2,3,0,1]
    const float s1 = v1 + dpp<0x4e>(v1), s3 = v3 + dpp<0x4e>(v3);
    const float w0 = b1 ? s2 : s0, w1 = b1 ? s3 : s1;
    const float r0 = w0 + dpp<0xb1>(w0), r1 = w1 + dpp<0xb1>(w1);   // quad_perm [1,0,3,2]
    return b0 ? r1 : r0;
}

// ---------------------------------------------------------------- math
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// softplus(x) = max(x, 0) + ln(1 + w), w = e^{-|x|} in (0, 1], with the
// hardware exp2 and log2. Forming v = 1 + w rounds w by r = (v - 1) - w
// (exact in fp32: v - 1 is exact for v in [1, 2], and so is the difference of
// the two nearby values), and ln(v) = ln(1 + w) + r / v. Subtracting r
// leaves an error of |r| w / v <= 2^-24 w, i.e. 2^-24 relative to ln(1 + w).
__device__ __forceinline__ float softplus_f(float x) {
    const float w = __builtin_amdgcn_exp2f(-__builtin_fabsf(x) * kLog2e);
    const float v = 1.f + w;
    const float r = (v - 1.f) - w;
    return fmaf(kLn2, __builtin_amdgcn_logf(v), fmaxf(x, 0.f) - r);
}
// silu(z) = z * sigmoid(z) = z / (1 + e^{-z})
__device__ __forceinline__ float silu_f(float z) {
    return z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// Workgroups are dispatched to the 8 XCDs (each with its own L2) round-robin
// by linear id. Renumber them so that every XCD receives one contiguous range
// of (batch, channel-group) ids: the workgroups that share a batch's B and C
// then mostly share one L2. A bijection on [0, G): XCD x gets the linear ids
// x, x+8, ..., which map to the range starting at x*(G/8) + min(x, G%8).
constexpr uint32_t kXcds = 8;
__device__ __forceinline__ void xcd_block(uint32_t& cg, uint32_t& bb) {
    const uint32_t G = gridDim.x * gridDim.y;
    const uint32_t lin = blockIdx.x + blockIdx.y * gridDim.x;
    const uint32_t x = lin % kXcds, k = lin / kXcds;
    const uint32_t q = G / kXcds, r = G % kXcds;
    const uint32_t v = x * q + (x < r ? x : r) + k;
    cg = v % gridDim.x;
    bb = v / gridDim.x;
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
//   1-D     : 16 channels, one direction (args.reverse)
//   Vim     : 8 channels x {forward, backward}; rows 2c and 2c+1 of channel c
//   cross-4 : 4 channels x the four VMamba orders. Waves 0-1 hold the
//             row-major pairs (k = 0 forward, 1 reverse) of channels 0-1 and
//             2-3, waves 2-3 the column-major pairs (k = 2, 3); within a
//             wave rows 2c' and 2c'+1 are one channel's pair.
// A direction and its reverse form a pair that visits every token at scan
// steps t and L-1-t; the two rows of a pair share one wave. The column-major
// pair reads u and delta from copies transposed to column-major order (a
// pre-pass), so its token at step t is entry t (or L-1-t) of the copy, read
// as contiguously as the row-major pair's; its partial sums stay in that
// order and are transposed back when the workgroup merges the pairs.
//
// Loop over blocks of 16 tokens. Global loads run two blocks ahead (raw
// bits in registers), the B/C tile of the next block is written to the other
// LDS buffer at the end of each step, and the per-step barrier orders LDS
// only. For the pair merge every block step is one of three phases:
//   steps < F : every token of the step is the first of its two visits
//               (forward token t < L/2, backward token > L/2): store y_k as
//               an fp32 partial sum;
//   step F    : the steps share tokens: forward stores, a fence, and the
//               backward row finishes the shared ones;
//   steps > F : every token is the second visit: add the partial sum
//               (prefetched one step ahead) and finish the token,
// with F = (L-1) / 32. The only global-memory fence is in step F; partial
// sums are read only after it. Vim finishes a token by gating and storing
// y; the cross-scan stores the pair's sum, and after the loop the workgroup
// adds its two pairs' sums, gates and stores y.
//
// CHUNK (Vim with shared inputs): the sequence is cut into a.nchunk chunks of
// whole 32-token tiles and each workgroup scans one chunk c, tokens
// [s_c, e_c), in both directions, as above over that sub-sequence. Its rows
// start from the states the directions carry into the chunk: the forward
// direction's state after tokens [0, s_c), the backward direction's after
// tokens [e_c, L) taken from L-1 down. A first phase computes them in the
// workgroup: a row scans a piece of that prefix or suffix from h = 0 (no
// read-out) and keeps the piece's aggregate (P_n = prod_t exp(delta_t A_n) =
// exp(A_n sum_t delta_t), h_n = its end state from 0). Aggregates compose
// associatively in scan order, (P1, h1) o (P2, h2) = (P1 P2, P2 h1 + h2);
// a prefix or suffix split over the channel's two rows is combined across
// them with one lane swizzle. The channel's rows take:
//   middle chunk   : row 0 the prefix (forward), row 1 the suffix (backward);
//   first chunk    : the suffix, split: row 0 the part next to L (scanned
//                    first), row 1 the rest, which then combines both;
//   last chunk     : the prefix, split: row 1 the part from token 0, row 0
//                    the rest, which then combines both.
template <typename T, int MODE, bool GATE, bool SOFTPLUS, bool CONV = false, bool CKPT = false,
          bool ZOH = false, bool CHUNK = false, bool GLDS = false, bool PLDS = false>
__global__ __launch_bounds__(kThreads) void rowscan_kernel(const ScanArgs a) {
    static_assert(!CONV || MODE == kModeVim, "the conv front end is Vim's");
    // GLDS (cross-scan grids that fit, vs::cross4_grid_in_lds): the
    // workgroup copies its channels' u and delta into LDS in column-major
    // order, and the column-major orders read them there instead of from
    // transposed copies in the workspace
    static_assert(!GLDS || MODE == kModeCross4, "the LDS grid serves the cross-scan's column orders");
    // PLDS (Vim sequences that fit, vs::vim_partial_lds_bytes): a channel's
    // forward and backward rows, which share a wave, hand each other their
    // partial sums through dynamic LDS, [channel][token] after a guard,
    // instead of the fp32 buffer in global memory
    static_assert(!PLDS || (MODE == kModeVim && !CONV && !CKPT && !ZOH),
                  "partial sums in LDS: the Vim scan without checkpoints");
    static_assert(!CHUNK || (MODE == kModeVim && !CONV && !CKPT && !ZOH),
                  "chunks: the plain Vim scan only");
    // CKPT (the gradient's forward pass): store every row's state at each
    // block start and the merged ungated sum in the partial buffer (fp32);
    // y (gated) is written as well when it is given
    static_assert(!CKPT || MODE == kModeVim, "checkpoints: Vim only");
    // ZOH: the exact zero-order hold B_bar = (exp(delta A) - 1) / A B ("Discretization
    // via Zero-Order Hold (ZOH)") in place of delta B
    static_assert(!(ZOH && CKPT), "the gradient uses delta B");
    constexpr int kDirs = MODE == kModeVim ? 2 : (MODE == kModeCross4 ? 4 : 1);
    constexpr int kChPerWg = 16 / kDirs;
    static_assert(MODE != kModeVim || kChPerWg == vs::kVimChPerWg, "the host sizes the LDS partial sums");
    static_assert(MODE != kModeCross4 || kChPerWg == vs::kCrossChPerWg, "the host sizes the LDS grid");
    constexpr int kSides = kDirs;              // one B/C tile per direction
    // B/C tiles of kPairTok tokens (two blocks; measured faster than four
    // for short and long sequences alike), rows padded to kPairPad floats,
    // which keeps the b128 row reads of 16 lanes on distinct banks. Two tile
    // buffers.
    constexpr int kPairTok = 32;
    constexpr int kPairPad = kPairTok + 4;
    constexpr int kBpt = kPairTok / kBlockTok;              // blocks per tile
    constexpr int kBufFloats = kSides * 2 * kRowLanes * kPairPad;
    __shared__ __attribute__((aligned(16))) float tile_mem[2 * kBufFloats];
    float (&tile)[2][kSides][2][kRowLanes][kPairPad] =
        *reinterpret_cast<float (*)[2][kSides][2][kRowLanes][kPairPad]>(tile_mem);

    const int tid = threadIdx.x;
    const int lane = tid & (kWaveLanes - 1);
    const int row_in_wg = tid >> 4;           // 0..15
    const int n = lane & (kRowLanes - 1);     // state index, also token slot
    // the wave index is uniform: reading it through readfirstlane lets the
    // per-wave tensor choices below live in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool colpair = MODE == kModeCross4 && wave >= 2;
    int dir, ch;
    if (MODE == kModeCross4) {
        const int r4 = row_in_wg & 3;
        ch = ((wave & 1) << 1) | (r4 >> 1);
        dir = (colpair ? 2 : 0) | (r4 & 1);
    } else {
        dir = row_in_wg % kDirs;
        ch = row_in_wg / kDirs;
    }
    uint32_t cg, bb;
    xcd_block(cg, bb);
    // grid.y enumerates (batch, chunk), chunk fastest
    const int nchunk = CHUNK ? a.nchunk : 1;
    const int chunk = CHUNK ? static_cast<int>(bb % static_cast<uint32_t>(nchunk)) : 0;
    const int64_t b = CHUNK ? bb / static_cast<uint32_t>(nchunk) : bb;
    const int64_t d0 = static_cast<int64_t>(cg) * kChPerWg + ch;
    const bool active = d0 < a.dim;
    const int64_t d = active ? d0 : 0;
    const int Lseq = static_cast<int>(a.L);
    // chunk c: tiles [c T / K, (c + 1) T / K) of the T = ceil(L / 32) tiles
    const int ntile_seq = (Lseq + kPairTok - 1) / kPairTok;
    auto chunk_start = [&](int k) {
        const int t = static_cast<int>(static_cast<int64_t>(ntile_seq) * k / nchunk) * kPairTok;
        return t < Lseq ? t : Lseq;
    };
    const int tok0 = CHUNK ? chunk_start(chunk) : 0;           // this workgroup's first token
    const int L = CHUNK ? chunk_start(chunk + 1) - tok0 : Lseq; // and its token count
    const int nblk = CHUNK ? (L + kBlockTok - 1) / kBlockTok : a.nblk;
    const bool rev = MODE == kMode1D ? a.reverse != 0 : (dir & 1) != 0;
    const int pside = dir & 1;                // position within the pair

    // per-row parameters
    const int64_t prow = (MODE == kMode1D ? 0 : dir * a.dim) + d;
    const float An = (active && n < a.dstate) ? a.A[prow * a.dstate + n] : 0.f;
    const float A2 = An * kLog2e;
    const float rA = ZOH ? 1.f / An : 0.f;    // A = 0 only ever takes the series below
    const float Dk = (active && a.Dskip) ? a.Dskip[prow] : 0.f;
    const float bias = (active && a.dt_bias) ? a.dt_bias[prow] : 0.f;
    // the other direction's A and dt_bias (a chunked row may scan a piece of
    // the other direction's prefix or suffix first)
    float A2_other = 0.f, bias_other = 0.f;
    if (CHUNK && active) {
        const int64_t orow = (1 - dir) * a.dim + d;
        A2_other = n < a.dstate ? a.A[orow * a.dstate + n] * kLog2e : 0.f;
        bias_other = a.dt_bias ? a.dt_bias[orow] : 0.f;
    }
    // Vim front end: each branch's u = silu(b + w0 x[q-1] + w1 x[q] + w2 x[q+1])
    // over its own sequence order q, with zeros past the ends ("1. Forward
    // Branch", "2. Backward Branch (Reverse sequence)"). In token order the
    // backward branch's left neighbour is token p+1, so its taps are
    // mirrored: cw_l multiplies x[p-1], cw_r multiplies x[p+1].
    float cw_l = 0.f, cw_c = 0.f, cw_r = 0.f, cw_b = 0.f;
    if (CONV && active) {
        const float* w = a.conv_w + prow * 3;
        cw_l = rev ? w[2] : w[0];
        cw_c = w[1];
        cw_r = rev ? w[0] : w[2];
        cw_b = a.conv_b ? a.conv_b[prow] : 0.f;
    }
    // Every tensor is addressed as its scalar base address plus a 32-bit
    // byte offset (tensors stay below 4 GiB), which keeps per-lane 64-bit
    // address arithmetic out of the loop.
    constexpr uint32_t kEs = sizeof(T);
    const uint32_t rowoff = static_cast<uint32_t>((b * a.dim + d) * a.L);
    const char* __restrict__ ub = static_cast<const char*>(colpair ? a.uT : a.u);
    const char* __restrict__ db = static_cast<const char*>(colpair ? a.deltaT : a.delta);
    const char* __restrict__ zb = static_cast<const char*>(a.z);
    char* __restrict__ yb = static_cast<char*>(a.y);
    char* __restrict__ pb = reinterpret_cast<char*>(colpair ? a.partial2 : a.partial);
    auto act_at = [&](const char* base, int p) {
        return ld_raw(reinterpret_cast<const T*>(base + (rowoff + static_cast<uint32_t>(p)) * kEs), 0);
    };
    const uint32_t u_row = rowoff + (MODE == kModeVim && rev ? a.dir_off : 0u);
    const uint32_t dl_row = u_row;
    auto act_row = [&](const char* base, uint32_t row, int p) {
        return ld_raw(reinterpret_cast<const T*>(base + (row + static_cast<uint32_t>(p)) * kEs), 0);
    };
    auto part_at = [&](int p) {
        return reinterpret_cast<float*>(pb + (rowoff + static_cast<uint32_t>(p)) * 4u);
    };
    auto y_at = [&](int p) {
        return reinterpret_cast<T*>(yb + (rowoff + static_cast<uint32_t>(p)) * kEs);
    };
    // Vim token addressing (every Vim form): a wave's two
    // channels are adjacent rows of [batch][dim][L], so one buffer descriptor
    // per tensor covers the wave, and a lane's token of block blk is one byte
    // offset ob0 + blk * ob_inc, never clamped: past either end of the
    // sequence it falls in the wave's other row (a token no step uses) or
    // outside the descriptor, where loads return 0. Loads that a block does
    // not need (the gate and the partial sum before the token's second
    // visit) take an out-of-range scalar offset and read nothing.
    constexpr bool kRun = MODE == kModeVim;
    constexpr int kOob = 0x40000000;
    const int64_t wave_d0 = static_cast<int64_t>(cg) * kChPerWg + 2 * wave;
    const int64_t wave_left = a.dim - wave_d0;
    const int64_t wave_nch = wave_left < 0 ? 0 : (wave_left > 2 ? 2 : wave_left);
    const size_t wave_base = static_cast<size_t>((b * a.dim + (wave_nch > 0 ? wave_d0 : 0)) * a.L);
    const uint32_t wave_el = static_cast<uint32_t>(wave_nch * a.L);
    auto wave_rsrc = [&](const void* base, uint32_t es, uint32_t extra_el) {
        return __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(static_cast<const char*>(base)) + wave_base * es, 0,
            static_cast<int>((wave_el + extra_el) * es), 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t rs_u = wave_rsrc(a.u, kEs, a.dir_off);
    const __amdgpu_buffer_rsrc_t rs_dl = wave_rsrc(a.delta, kEs, a.dir_off);
    const __amdgpu_buffer_rsrc_t rs_z = wave_rsrc(GATE ? a.z : a.u, kEs, 0u);
    // a checkpointing pass without y gets a descriptor that covers nothing:
    // its y stores are dropped
    const bool y_none = CKPT && a.y == nullptr;
    const __amdgpu_buffer_rsrc_t rs_y = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(y_none ? a.u : a.y)) + wave_base * kEs, 0,
        y_none ? 0 : static_cast<int>(wave_el * kEs), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_p = wave_rsrc(a.partial, 4u, 0u);
    // an inactive channel's lanes land past the wave's rows (no store ever
    // uses them)
    const int lane_rel = static_cast<int>((d0 - wave_d0) * a.L);
    const int ob0 = (lane_rel + tok0 + (rev ? L - 1 - n : n)) * static_cast<int>(kEs);
    const int ob_inc = (rev ? -kBlockTok : kBlockTok) * static_cast<int>(kEs);
    // u and delta of a backward row (per-direction inputs)
    const int o_dir = rev ? static_cast<int>(a.dir_off * kEs) : 0;
    // (CONV, never chunked) byte offsets of the sequence's first and last
    // tokens in this lane's row
    const int conv_lo = lane_rel * static_cast<int>(kEs);
    const int conv_hi = (lane_rel + Lseq - 1) * static_cast<int>(kEs);
    auto rload = [&](__amdgpu_buffer_rsrc_t r, int off, int soff) VS_INLINE {
        if constexpr (sizeof(T) == 2)
            return static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0));
        else
            return static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0));
    };
    auto rstore = [&](__amdgpu_buffer_rsrc_t r, int off, float v) VS_INLINE {
        if constexpr (sizeof(T) == 2)
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v)), r, off, 0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
    };
    // byte offset of a token's fp32 partial sum from its activation offset
    auto poff = [&](int ob) { return ob * static_cast<int>(4 / kEs); };

    // ---- B/C staging, one tile per kPairTok tokens. The tile's rows are
    // (side, B|C, state); a row's entries are 16-byte chunks (8
    // bf16 or 4 fp32 entries) that lie contiguously in memory, in token order
    // or, for a side that reads token L-1-t, in reverse order. Thread tid
    // loads chunks tid, tid + 256, ... with one 16-byte load each (rows start
    // at any 2-byte boundary; the target handles unaligned global loads), at
    // a per-lane offset that steps by one tile per tile. A last tile that
    // the sequence does not fill is read entry by entry, clamped, when its
    // turn comes. Vim's two sides read the shared B/C at tokens t and L-1-t;
    // each cross-scan direction reads its own B/C, stored in its scan order.
    //
    // The store builds each fp32 tile entry with one byte permute (v_perm)
    // of two loaded words, the word for token order and the word for reverse
    // order, so that one selector per chunk does the bf16 widening, the
    // reversal and, for rows of states >= dstate, the zero fill (those state
    // lanes then never change). fp32 data that is never reversed (the
    // cross-scan) is stored as loaded, and the rows of states >= dstate are
    // zeroed once and never written.
    constexpr bool kRawStore = sizeof(T) == 4 && MODE == kModeCross4;
    constexpr int kTpc = 16 / static_cast<int>(sizeof(T));      // entries per chunk
    constexpr int kCpr = kPairTok / kTpc;                       // chunks per row
    constexpr int kChunks = kSides * 2 * kRowLanes * kCpr;
    constexpr int kCpt = (kChunks + kThreads - 1) / kThreads;   // chunks per thread
    static_assert(kRowLanes * kCpr * 2 % kWaveLanes == 0, "a wave's chunks share one side");
    // selectors: byte i of the result is byte sel[i] of {S0 (bytes 4-7) : S1
    // (bytes 0-3)}, 0x0c gives 0. S1 holds the token-order word, S0 the
    // reverse-order one.
    constexpr uint32_t kSelZero = 0x0c0c0c0cu;
    constexpr uint32_t kSelFwdX = sizeof(T) == 2 ? 0x01000c0cu : 0x03020100u;   // S1 low half / word
    constexpr uint32_t kSelFwdY = sizeof(T) == 2 ? 0x03020c0cu : 0x03020100u;   // S1 high half / word
    constexpr uint32_t kSelRevX = sizeof(T) == 2 ? 0x07060c0cu : 0x07060504u;   // S0 high half / word
    constexpr uint32_t kSelRevY = sizeof(T) == 2 ? 0x05040c0cu : 0x07060504u;   // S0 low half / word
    const int64_t bc_dirs = MODE == kModeCross4 ? 4 : (MODE == kModeVim && a.bc_per_dir ? 2 : 1);
    const char* __restrict__ Bb = static_cast<const char*>(a.B);
    const char* __restrict__ Cb = static_cast<const char*>(a.C);
    // chunk j of every thread in a wave lies in rows of one (side, B|C) tile,
    // so the tensor it reads is uniform per wave: one buffer descriptor over
    // this batch's B or C
    const uint32_t bc_batch_el = static_cast<uint32_t>(bc_dirs * a.dstate * a.L);
    __amdgpu_buffer_rsrc_t csrc[kCpt];
    uint32_t crow[kCpt];        // row start within the batch (entries)
    int ccol[kCpt];             // first token of the chunk within the tile
    bool cin[kCpt];             // the thread has this chunk (uniform per wave)
    bool crev[kCpt];            // reverse token order (uniform per wave)
    uint32_t cselx[kCpt], csely[kCpt];
    bool cok[kCpt];             // the chunk's state row is < dstate
    int cdst[kCpt];             // tile_mem index of the chunk in buffer 0
    int ctok0[kCpt], clen[kCpt];    // the side's token range (uniform per wave)
    // byte offset of the chunk's 16 bytes in tile 0, and its step per tile
    // (negative in reverse order; uniform per wave)
    int cbase[kCpt], cinc[kCpt];
    // A side s reads tokens [sd_tok0[s], sd_tok0[s] + sd_len[s]) in token
    // order, or from the top down when sd_rev[s]; with_c = false stages B only.
    auto stage_setup = [&](const int (&sd_tok0)[kSides], const int (&sd_len)[kSides],
                           const bool (&sd_rev)[kSides], bool with_c) VS_INLINE {
#pragma unroll
        for (int j = 0; j < kCpt; ++j) {
            const int c0 = tid + j * kThreads;
            const int c = c0 < kChunks ? c0 : 0;
            const int row = c / kCpr, k = c % kCpr;
            const int q = row / kRowLanes, srow = row % kRowLanes;
            const int side = q >> 1;
            const bool ok_row = srow < a.dstate;
            const int64_t dsel = MODE == kModeCross4 ? side : (MODE == kModeVim && a.bc_per_dir ? side : 0);
            const bool isC = __builtin_amdgcn_readfirstlane(q & 1) != 0;
            cin[j] = (kChunks % kThreads == 0 || __builtin_amdgcn_readfirstlane(c0 < kChunks ? 1 : 0) != 0) &&
                     (with_c || !isC);
            csrc[j] = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<char*>(isC ? Cb : Bb) + static_cast<size_t>(b) * bc_batch_el * kEs, 0,
                static_cast<int>(bc_batch_el * kEs), 0x00020000);
            crow[j] = static_cast<uint32_t>((dsel * a.dstate + (ok_row ? srow : 0)) * a.L);
            ccol[j] = k * kTpc;
            const bool rv = sd_rev[side];
            crev[j] = MODE != kModeCross4 && __builtin_amdgcn_readfirstlane(rv ? 1 : 0) != 0;
            ctok0[j] = sd_tok0[side];
            clen[j] = sd_len[side];
            cok[j] = ok_row;
            cselx[j] = !ok_row ? kSelZero : (rv ? kSelRevX : kSelFwdX);
            csely[j] = !ok_row ? kSelZero : (rv ? kSelRevY : kSelFwdY);
            cdst[j] = ((side * 2 + (q & 1)) * kRowLanes + srow) * kPairPad + k * kTpc;
            const uint32_t first0 = static_cast<uint32_t>(ctok0[j]) +
                                    (crev[j] ? static_cast<uint32_t>(clen[j] - kTpc - ccol[j])
                                             : static_cast<uint32_t>(ccol[j]));
            cbase[j] = static_cast<int>((crow[j] + first0) * kEs);
            cinc[j] = (crev[j] ? -kPairTok : kPairTok) * static_cast<int>(kEs);
        }
    };
    // The tile `pair` of chunk j's side, entry by entry and clamped into the
    // side's range: entry i of the chunk in memory order holds scan step
    // t0 + i (t0 + kTpc - 1 - i when reversed); steps past the range repeat
    // its last step.
    auto stage_entries = [&](int pair, int j) VS_INLINE {
        const int t0 = pair * kPairTok + ccol[j];
        uint32_t e[kTpc];
#pragma unroll
        for (int i = 0; i < kTpc; ++i) {
            const int t = t0 + (crev[j] ? kTpc - 1 - i : i);
            const int tc = t < clen[j] ? t : clen[j] - 1;
            const int tok = ctok0[j] + (crev[j] ? clen[j] - 1 - tc : tc);
            const int off = static_cast<int>((crow[j] + static_cast<uint32_t>(tok)) * kEs);
            e[i] = sizeof(T) == 2 ? __builtin_amdgcn_raw_buffer_load_b16(csrc[j], off, 0, 0)
                                  : __builtin_amdgcn_raw_buffer_load_b32(csrc[j], off, 0, 0);
        }
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[i] = sizeof(T) == 2 ? (e[2 * i] | (e[2 * i + 1] << 16)) : e[i];
            // materialise here: packing at the use inside the loop would
            // have to wait for every load then in flight
            asm volatile("" : "+v"(w[i]));
        }
        return make_uint4(w[0], w[1], w[2], w[3]);
    };
    {
        int sd_tok0[kSides], sd_len[kSides];
        bool sd_rev[kSides];
#pragma unroll
        for (int sd = 0; sd < kSides; ++sd) {
            sd_tok0[sd] = tok0;
            sd_len[sd] = L;
            sd_rev[sd] = MODE == kModeVim ? sd == 1 : (MODE == kMode1D ? a.reverse != 0 : false);
        }
        stage_setup(sd_tok0, sd_len, sd_rev, true);
    }
    // whole tiles with one 16-byte load per chunk at its running offset; a
    // last tile that the side's range does not fill is read entry by entry
    // (once per scan, in a branch that is uniform per wave)
    auto stage_load = [&](int pair, uint4 (&raw)[kCpt]) VS_INLINE {
#pragma unroll
        for (int j = 0; j < kCpt; ++j) {
            if (!cin[j]) continue;
            if ((pair + 1) * kPairTok <= clen[j])
                raw[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       csrc[j], cbase[j] + pair * cinc[j], 0, 0));
            else
                raw[j] = stage_entries(pair, j);
        }
    };
    auto stage_store = [&](int buf, const uint4 (&raw)[kCpt]) VS_INLINE {
#pragma unroll
        for (int j = 0; j < kCpt; ++j) {
            if (!cin[j]) continue;
            float4* d4 = reinterpret_cast<float4*>(&tile_mem[cdst[j] + buf * kBufFloats]);
            if constexpr (kRawStore) {
                if (cok[j])
                    d4[0] = make_float4(__uint_as_float(raw[j].x), __uint_as_float(raw[j].y),
                                        __uint_as_float(raw[j].z), __uint_as_float(raw[j].w));
                continue;
            }
            const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
            // tile columns 2d, 2d + 1 of the chunk: token order takes them from
            // word d (bf16: its low and high halves) or words 2d, 2d + 1
            // (fp32); reverse order from word 3 - d (high, low) or words
            // 3 - 2d, 2 - 2d
            float f[kTpc];
#pragma unroll
            for (int d = 0; d < kTpc / 2; ++d) {
                const uint32_t fx = sizeof(T) == 2 ? w[d] : w[2 * d];
                const uint32_t fy = sizeof(T) == 2 ? w[d] : w[2 * d + 1];
                const uint32_t rx = sizeof(T) == 2 ? w[3 - d] : w[3 - 2 * d];
                const uint32_t ry = sizeof(T) == 2 ? w[3 - d] : w[2 - 2 * d];
                f[2 * d] = __uint_as_float(__builtin_amdgcn_perm(rx, fx, cselx[j]));
                f[2 * d + 1] = __uint_as_float(__builtin_amdgcn_perm(ry, fy, csely[j]));
            }
#pragma unroll
            for (int i = 0; i < kTpc / 4; ++i)
                d4[i] = make_float4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]);
        }
    };
    if (kRawStore) {
        for (int i = tid; i < 2 * kBufFloats; i += kThreads)
            if ((i / kPairPad) % kRowLanes >= a.dstate) tile_mem[i] = 0.f;
    }

    // ---- this lane's token of a block (slot n), clamped into the sequence;
    // for the column-major pair it indexes the transposed copies
    auto tok_pos = [&](int blk) {
        const int t = blk * kBlockTok + n;
        const int tc = t < L ? t : L - 1;
        return tok0 + (rev ? L - 1 - tc : tc);
    };

    // ---- this lane's token of a block; unconditional loads on a valid
    // index so that they can all be in flight together.
    const int Fstep = MODE != kMode1D ? (L - 1) / (2 * kBlockTok) : -1;
    // raw entries at their own width: a bf16 entry held zero-extended would
    // be re-masked where the loop carries it, which waits for its load
    using Raw = std::conditional_t<sizeof(T) == 2, uint16_t, uint32_t>;
    struct Tok { Raw u, dl, z, ul, ur; int p; };
    // the LDS grid (GLDS): [u | delta][channel][column-major token], sized at
    // launch (2 x kChPerWg x L entries)
    extern __shared__ __attribute__((aligned(16))) char glds_bytes[];
    Raw* const glds = reinterpret_cast<Raw*>(glds_bytes);
    // PLDS: byte offset of this lane's token of block blk in the LDS partial
    // sums, lp0 + blk * lp_inc (past either end of the row it falls in a
    // guard or a neighbour row, and only stores of valid tokens are made)
    const int lp0 = (vs::kPartLdsGuard + ch * L + (rev ? L - 1 - n : n)) * 4;
    const int lp_inc = (rev ? -kBlockTok : kBlockTok) * 4;
    auto lpart = [&](int blk) { return reinterpret_cast<float*>(glds_bytes + lp0 + blk * lp_inc); };
    auto tok_load = [&](int blk, Tok& k) VS_INLINE {
        if constexpr (kRun) {
            // p holds the token's byte offset within the wave's rows
            const int ob = ob0 + blk * ob_inc;
            k.p = ob;
            k.u = static_cast<Raw>(rload(rs_u, ob + o_dir, 0));
            if (CONV) {   // the neighbours (masked at the sequence ends)
                k.ul = static_cast<Raw>(rload(rs_u, ob + o_dir - static_cast<int>(kEs), 0));
                k.ur = static_cast<Raw>(rload(rs_u, ob + o_dir + static_cast<int>(kEs), 0));
            }
            k.dl = static_cast<Raw>(rload(rs_dl, ob + o_dir, 0));
            if (GATE) k.z = static_cast<Raw>(rload(rs_z, ob, blk >= Fstep ? 0 : kOob));
            return;
        }
        const int p = tok_pos(blk);
        k.p = p;
        if constexpr (GLDS) {
            if (colpair) {          // uniform per wave
                k.u = glds[ch * Lseq + p];
                k.dl = glds[(kChPerWg + ch) * Lseq + p];
                return;
            }
        }
        k.u = act_row(ub, u_row, p);
        if (CONV) {   // the neighbours (clamped; masked where they fall outside)
            k.ul = act_row(ub, u_row, p > 0 ? p - 1 : 0);
            k.ur = act_row(ub, u_row, p < Lseq - 1 ? p + 1 : Lseq - 1);
        }
        k.dl = act_row(db, dl_row, p);
        // z is needed only by the visit that finishes the token; other
        // blocks load entry 0 of the row (one cached line) instead of
        // branching, which would stall on the in-flight registers. The
        // cross-scan gates after the loop.
        if (GATE && MODE != kModeCross4)
            k.z = act_at(zb, (MODE != kModeVim || blk >= Fstep) ? p : 0);
    };

    const int npair = (nblk + kBpt - 1) / kBpt;
    uint4 sr[kCpt];
    // token data rotates through kTokAhead + 1 register sets, so that the
    // loads of kTokAhead blocks are in flight while one block is computed
    // (deeper prefetch measured no faster)
    constexpr int kRing = kTokAhead + 1;
    static_assert(kRing % kBpt == 0, "a loop trip covers whole tiles");
    Tok tk[kRing];
    auto wg_barrier = [&]() VS_INLINE {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };

    float h = 0.f;
    // ---- chunks: the states the two directions carry into this chunk
    if constexpr (CHUNK) if (nchunk > 1) {
        const bool pre = chunk > 0, suf = chunk < nchunk - 1;          // uniform
        const int e_tok = tok0 + L;
        // side s (row parity) scans tokens [pa_s, pa_s + pl_s) in direction
        // pd_s (1: from the top down)
        int pa0, pl0, pd0, pa1, pl1, pd1;
        const bool split = !(pre && suf);
        if (!split) {
            pa0 = 0; pl0 = tok0; pd0 = 0;                      // the prefix, forward
            pa1 = e_tok; pl1 = Lseq - e_tok; pd1 = 1;          // the suffix, backward
        } else {
            // one job [ja, jb) in direction jd, split in two pieces: the near
            // one is scanned first, the far one (a whole number of tiles)
            // after it
            const int ja = pre ? 0 : e_tok, jb = pre ? tok0 : Lseq, jd = pre ? 0 : 1;
            const int jl = jb - ja;
            const int far_len = ((jl + kPairTok - 1) / kPairTok / 2) * kPairTok;
            const int near_len = jl - far_len;
            const int near_a = jd == 0 ? ja : jb - near_len;
            const int far_a = jd == 0 ? ja + near_len : ja;
            // the far piece goes to the row of direction jd, which combines
            // both pieces into its own carry; the other row starts the chunk
            // at a sequence end, from zero
            pa0 = jd == 0 ? far_a : near_a;
            pl0 = jd == 0 ? far_len : near_len;
            pa1 = jd == 0 ? near_a : far_a;
            pl1 = jd == 0 ? near_len : far_len;
            pd0 = pd1 = jd;
        }
        const int mpa = pside ? pa1 : pa0, mpl = pside ? pl1 : pl0;
        const int mlen = mpl > 0 ? mpl : 1;             // an empty piece reads a valid token
        const bool mrev = (pside ? pd1 : pd0) != 0;
        const bool own_dir = (pside ? pd1 : pd0) == dir;
        const float A2a = own_dir ? A2 : A2_other;
        const float bias_a = own_dir ? bias : bias_other;
        {
            const int sd_tok0[kSides] = {pa0, pa1};
            const int sd_len[kSides] = {pl0 > 0 ? pl0 : 1, pl1 > 0 ? pl1 : 1};
            const bool sd_rev[kSides] = {pd0 != 0, pd1 != 0};
            stage_setup(sd_tok0, sd_len, sd_rev, false);
        }
        const int lmax = pl0 > pl1 ? pl0 : pl1;
        const int nblk_a = (lmax + kBlockTok - 1) / kBlockTok;
        const int npair_a = (nblk_a + kBpt - 1) / kBpt;
        // the piece's tokens through the wave's descriptors, as the main scan
        // reads its own: one byte offset per lane, linear in the block and
        // never clamped (past the piece it reads a token no valid step uses,
        // or nothing outside the wave's rows)
        const int oa0 = (lane_rel + mpa + (mrev ? mlen - 1 - n : n)) * static_cast<int>(kEs);
        const int oa_inc = (mrev ? -kBlockTok : kBlockTok) * static_cast<int>(kEs);
        auto tok_load_a = [&](int blk, Tok& k) VS_INLINE {
            const int ob = oa0 + blk * oa_inc;
            k.u = static_cast<Raw>(rload(rs_u, ob, 0));
            k.dl = static_cast<Raw>(rload(rs_dl, ob, 0));
        };
        stage_load(0, sr);
        stage_store(0, sr);
        Unroll<kTokAhead>::run([&](auto ic) {
            constexpr int k = decltype(ic)::value;
            tok_load_a(k < nblk_a ? k : nblk_a - 1, tk[k]);
        });
        wg_barrier();
        float sdl = 0.f;          // this lane's share of the piece's sum of delta
        auto step_a = [&](const int blk, Tok& cur, Tok& nxt) VS_INLINE {
            const int buf = (blk / kBpt) & 1;
            const int half = blk % kBpt;
            if (half == 0) {
                const int pair = blk / kBpt;
                stage_load(pair + 1 < npair_a ? pair + 1 : pair, sr);
            }
            tok_load_a(blk + kTokAhead < nblk_a ? blk + kTokAhead : nblk_a - 1, nxt);
            const bool ok = active && n < mpl - blk * kBlockTok;
            const float cu = from_raw<T>(cur.u);
            const float x = from_raw<T>(cur.dl) + bias_a;
            const float dlt = ok ? (SOFTPLUS ? softplus_f(x) : x) : 0.f;
            // the select keeps a non-finite value read past the piece (it may
            // be another channel's) out of the state
            const float du = ok ? dlt * cu : 0.f;
            sdl += dlt;
            const float4* Bt = reinterpret_cast<const float4*>(&tile[buf][pside][0][n][half * kBlockTok]);
            float Bv[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 bq = Bt[q];
                Bv[4 * q] = bq.x; Bv[4 * q + 1] = bq.y; Bv[4 * q + 2] = bq.z; Bv[4 * q + 3] = bq.w;
            }
            Unroll<16>::run([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                const float e = __builtin_amdgcn_exp2f(row_bcast<i>(dlt) * A2a);
                h = fmaf(e, h, row_bcast<i>(du) * Bv[i]);
            });
            // with no read-out, nothing else ties the unrolled steps
            // together: left free, the scheduler hoists the exps of later
            // blocks and the kernel needs 246 VGPRs (2 waves per SIMD)
            // instead of 81
            asm volatile("" : "+v"(h));
            if (half == kBpt - 1) {
                stage_store(buf ^ 1, sr);
                wg_barrier();
            }
        };
        int blk = 0;
        for (; blk + kTokAhead < nblk_a; blk += kRing) {
            Unroll<kRing>::run([&](auto ic) {
                constexpr int k = decltype(ic)::value;
                step_a(blk + k, tk[k], tk[(k + kTokAhead) % kRing]);
            });
        }
        Unroll<kTokAhead>::run([&](auto ic) {
            constexpr int k = decltype(ic)::value;
            if (blk + k < nblk_a) step_a(blk + k, tk[k], tk[(k + kTokAhead) % kRing]);
        });
        // every wave is past its last read of the tile buffers before the
        // chunk's own scan stages into them
        wg_barrier();
        if (split) {
            // the far row composes the near piece's aggregate with its own:
            // carry = P_far h_near + h_far, P_far = exp(A sum(delta)) over
            // the far piece. The near piece is the other row of the channel,
            // 16 lanes away in the same 32-lane half of the wave.
            float S = sdl;
            S += dpp<0x128>(S);                                  // row_ror:8
            S += dpp<0x124>(S);                                  // row_ror:4
            S += dpp<0x122>(S);                                  // row_ror:2
            S += dpp<0x121>(S);                                  // row_ror:1
            const float h_other = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(h), 0x401f));
            const bool far_row = own_dir;                        // the row of the job's direction
            h = far_row ? fmaf(__builtin_amdgcn_exp2f(A2a * S), h_other, h) : 0.f;
        }
        {
            int sd_tok0[kSides], sd_len[kSides];
            bool sd_rev[kSides];
#pragma unroll
            for (int sd = 0; sd < kSides; ++sd) {
                sd_tok0[sd] = tok0;
                sd_len[sd] = L;
                sd_rev[sd] = sd == 1;
            }
            stage_setup(sd_tok0, sd_len, sd_rev, true);
        }
    }

    if constexpr (GLDS) {
        // the workgroup's u and delta grids, read row by row (coalesced) and
        // written at their column-major index j H + i; a channel past dim
        // gets zeros
        const int Hg = a.H, Wg = a.W;
        const Raw* __restrict__ ug = static_cast<const Raw*>(a.u);
        const Raw* __restrict__ dg = static_cast<const Raw*>(a.delta);
        const int64_t dfirst = static_cast<int64_t>(cg) * kChPerWg;
        for (int e = tid; e < kChPerWg * Lseq; e += kThreads) {
            const int c = e / Lseq, r = e - c * Lseq;
            const int i = r / Wg, j = r - i * Wg;
            const bool okc = dfirst + c < a.dim;
            const size_t g = static_cast<size_t>(b * a.dim + (okc ? dfirst + c : 0)) * Lseq + r;
            const Raw uv = okc ? ug[g] : Raw(0), dv = okc ? dg[g] : Raw(0);
            glds[c * Lseq + j * Hg + i] = uv;
            glds[(kChPerWg + c) * Lseq + j * Hg + i] = dv;
        }
        wg_barrier();
    }
    stage_load(0, sr);
    stage_store(0, sr);
    Unroll<kTokAhead>::run([&](auto ic) {
        constexpr int k = decltype(ic)::value;
        tok_load(k < nblk ? k : nblk - 1, tk[k]);
    });
    wg_barrier();

    // checkpoints [batch][dim][direction][block][state]: the wave's four rows
    // are adjacent, so one descriptor covers them; an inactive channel's
    // lanes land past it and store nothing
    // (built in every form; only CKPT stores through it)
    const size_t ck_row_fl = static_cast<size_t>(nblk) * kRowLanes;
    const __amdgpu_buffer_rsrc_t rs_ck = __builtin_amdgcn_make_buffer_rsrc(
        a.ckpt + static_cast<size_t>(b * a.dim + (wave_nch > 0 ? wave_d0 : 0)) * 2 * ck_row_fl, 0,
        static_cast<int>(wave_nch * 2 * ck_row_fl * 4), 0x00020000);
    const int ck_off0 = static_cast<int>((static_cast<size_t>((d0 - wave_d0) * 2 + dir) * ck_row_fl + n) * 4);
    // One block step. `cur` holds this block's token data (loaded kTokAhead
    // steps earlier), `nxt` receives block blk + kTokAhead's; the loop below
    // rotates the sets so that no register of an in-flight load is ever
    // copied. The
    // first block of a tile issues the next tile's B/C loads, the last one
    // stores them to the other tile buffer and ends with the barrier.
    auto step = [&](const int blk, Tok& cur, Tok& nxt) VS_INLINE {
        const int buf = (blk / kBpt) & 1;
        const int half = blk % kBpt;
        const int p = cur.p;
        const bool ok = active && n < L - blk * kBlockTok;
        if constexpr (CKPT)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(h), rs_ck, ck_off0 + blk * (kRowLanes * 4), 0, 0);
        // the other direction's partial sum, for blocks after step F (it was
        // stored at step F or earlier, before F's fence); earlier blocks load
        // entry 0 of the row instead (unused) rather than branch. Issued
        // before the prefetch so that waiting for it does not wait for those.
        float part = 0.f;
        if (PLDS) {
            if (blk > Fstep) part = *lpart(blk);
        } else if (kRun) {  // agent-coherent (sc1), as the atomic load below
            part = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_p, poff(p), blk > Fstep ? 0 : kOob, 16));
        }
        else if (MODE != kMode1D)
            part = __hip_atomic_load(part_at(blk > Fstep ? p : 0), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
        // prefetch; near the end this reloads the last pair or block
        // (unused), which keeps the loads free of branches
        if (half == 0) {
            const int pair = blk / kBpt;
            stage_load(pair + 1 < npair ? pair + 1 : pair, sr);
        }
        tok_load(blk + kTokAhead < nblk ? blk + kTokAhead : nblk - 1, nxt);

        // delta and delta*u of this lane's token (zero in padding slots, which
        // then leave the state unchanged: exp(0) = 1 and no input)
        float cu = from_raw<T>(cur.u);
        if (CONV) {
            // (kRun: p is the token's byte offset, conv_lo and conv_hi those
            // of the row's first and last tokens)
            const bool has_l = kRun ? p > conv_lo : p > 0;
            const bool has_r = kRun ? p < conv_hi : p < Lseq - 1;
            const float xl = has_l ? from_raw<T>(cur.ul) : 0.f;
            const float xr = has_r ? from_raw<T>(cur.ur) : 0.f;
            cu = silu_f(fmaf(cw_l, xl, fmaf(cw_c, cu, fmaf(cw_r, xr, cw_b))));
        }
        const float x = from_raw<T>(cur.dl) + bias;
        const float dlt = ok ? (SOFTPLUS ? softplus_f(x) : x) : 0.f;
        const float du = dlt * cu;

        const int side = MODE == kMode1D ? 0 : dir;
        const float4* Bt = reinterpret_cast<const float4*>(&tile[buf][side][0][n][half * kBlockTok]);
        const float4* Ct = reinterpret_cast<const float4*>(&tile[buf][side][1][n][half * kBlockTok]);
        float Bv[16], Cv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 bb = Bt[q], cc = Ct[q];
            Bv[4 * q] = bb.x; Bv[4 * q + 1] = bb.y; Bv[4 * q + 2] = bb.z; Bv[4 * q + 3] = bb.w;
            Cv[4 * q] = cc.x; Cv[4 * q + 1] = cc.y; Cv[4 * q + 2] = cc.z; Cv[4 * q + 3] = cc.w;
        }
        float c[16];
        Unroll<16>::run([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            const float xl = row_bcast<i>(dlt) * A2;            // delta A log2(e)
            const float e = __builtin_amdgcn_exp2f(xl);
            float bu = row_bcast<i>(du);                        // B_bar u / B = delta u
            if (ZOH) {
                // (e - 1) / A u when |delta A| >= 1/2; below that the
                // subtraction cancels, so delta u phi(delta A) with
                // phi(x) = (e^x - 1) / x = sum x^k / (k + 1)!, to x^6
                const float xn = xl * kLn2;
                float phi = fmaf(xn, 1.f / 5040.f, 1.f / 720.f);
                phi = fmaf(xn, phi, 1.f / 120.f);
                phi = fmaf(xn, phi, 1.f / 24.f);
                phi = fmaf(xn, phi, 1.f / 6.f);
                phi = fmaf(xn, phi, 0.5f);
                phi = fmaf(xn, phi, 1.f);
                const float held = (e - 1.f) * rA * row_bcast<i>(cu);
                bu = fabsf(xn) < 0.5f ? bu * phi : held;
            }
            h = fmaf(e, h, bu * Bv[i]);
            c[i] = Cv[i] * h;
        });
        const float yk = fmaf(Dk, cu, row_transpose_sum(c, lane));
        const float gate = (GATE && MODE != kModeCross4) ? silu_f(from_raw<T>(cur.z)) : 1.f;
        // a token's second visit: Vim gates and stores y, the cross-scan
        // stores the pair's fp32 sum
        auto finish = [&](float sum, int pp) {
            if (kRun) {
                if (CKPT) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sum), rs_p, poff(pp), 0, 0);
                rstore(rs_y, pp, sum * gate);
            } else if (MODE == kModeCross4 || CKPT) {
                *part_at(pp) = sum;
            } else {
                st(y_at(pp), 0, sum * gate);
            }
        };

        if (MODE == kMode1D) {
            if (ok) st(y_at(p), 0, yk * gate);
        } else if (blk < Fstep) {
            if (ok) {
                if (PLDS) *lpart(blk) = yk;
                else if (kRun) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yk), rs_p, poff(p), 0, 0);
                else *part_at(p) = yk;
            }
        } else if (blk > Fstep) {
            if (ok) finish(yk + part, p);
        } else {
            // step F: tokens finished by the other direction in an earlier
            // step, or (forward row) shared with the backward row in this one.
            // It addresses the token by its index (once per scan).
            const int p = tok_pos(blk);
            const int t_self = blk * kBlockTok + n;
            const int blk_other = (L - 1 - t_self) / kBlockTok;
            const bool first = blk < blk_other || (blk == blk_other && pside == 0);
            // (PLDS) the token's entry in the LDS partial sums
            float* const lp = reinterpret_cast<float*>(glds_bytes) + vs::kPartLdsGuard + ch * L + (p - tok0);
            if (ok && first) {
                if (PLDS) *lp = yk;
                else __hip_atomic_store(part_at(p), yk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            // both rows are in this wave: with the sums in LDS, waiting for
            // its own LDS stores orders them before the reads below
            if (PLDS) __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup", "local");
            else __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
            if (ok && !first) {
                const float other = PLDS ? *lp : __hip_atomic_load(part_at(p), __ATOMIC_RELAXED,
                                                                   __HIP_MEMORY_SCOPE_AGENT);
                if (kRun) {
                    // finish through the element pointer as well
                    if (CKPT) *part_at(p) = yk + other;
                    if (!y_none) st(y_at(p), 0, (yk + other) * gate);
                } else {
                    finish(yk + other, p);
                }
            }
        }

        if (half == kBpt - 1) {
            stage_store(buf ^ 1, sr);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        }
    };

    // slot k of the ring holds block blk + k at the top of every trip.
    // The workgroups that share a CU drift apart (the arbiter issues the
    // oldest waves first), and the last one would run alone at the end. The
    // wave's issue priority steps down as it passes each quarter of its
    // blocks, so that lagging waves catch up and all finish together
    // (Vim-S 1024^2: 0.270 -> 0.250 ms; Vim-S 1248^2: 0.399 -> 0.372 ms).
    int blk = 0;
    __builtin_amdgcn_s_setprio(3);
    const int q1 = nblk / 4, q2 = nblk / 2, q3 = (3 * nblk) / 4;
    for (; blk + kTokAhead < nblk; blk += kRing) {
        if (blk >= q1 && blk < q1 + kRing) __builtin_amdgcn_s_setprio(2);
        if (blk >= q2 && blk < q2 + kRing) __builtin_amdgcn_s_setprio(1);
        if (blk >= q3 && blk < q3 + kRing) __builtin_amdgcn_s_setprio(0);
        Unroll<kRing>::run([&](auto ic) {
            constexpr int k = decltype(ic)::value;
            step(blk + k, tk[k], tk[(k + kTokAhead) % kRing]);
        });
    }
    Unroll<kTokAhead>::run([&](auto ic) {
        constexpr int k = decltype(ic)::value;
        if (blk + k < nblk) step(blk + k, tk[k], tk[(k + kTokAhead) % kRing]);
    });

    if constexpr (MODE == kModeCross4) {
        // every pair sum of the workgroup's channels is stored: y = (row-major
        // pair + column-major pair) * gate. The column-major sums are in
        // column-major order: 32 x 32 tiles of the grid pass through LDS,
        // read along columns and written along rows.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        // The tiles of all the workgroup's channels form one list, taken
        // kGroup at a time: the loads of a whole group are issued together,
        // then its column-major tiles are transposed through LDS, with two
        // barriers per group (one tile at a time left this phase waiting on
        // load latency: about 50 us per workgroup at 64 x 64).
        constexpr int kGroup = 8;
        static_assert(kGroup * kTr * kTrPad <= 2 * kBufFloats, "the transposition tiles fit the tile buffers");
        constexpr int kRpt = kTr * kTr / kThreads;           // tile rows per thread
        static_assert(kRpt * kThreads == kTr * kTr, "whole tile rows per thread");
        float (*tr)[kTr][kTrPad] = reinterpret_cast<float (*)[kTr][kTrPad]>(&tile_mem[0]);
        const char* __restrict__ p0 = reinterpret_cast<const char*>(a.partial);
        const char* __restrict__ p1 = reinterpret_cast<const char*>(a.partial2);
        const int H = a.H, Wd = a.W;
        const int tx = tid & (kTr - 1), ty = tid / kTr;
        const int tiles_w = (Wd + kTr - 1) / kTr, ntiles = tiles_w * ((H + kTr - 1) / kTr);
        const int64_t dfirst = static_cast<int64_t>(cg) * kChPerWg;
        const int nch = static_cast<int>(a.dim - dfirst < kChPerWg ? a.dim - dfirst : kChPerWg);
        const int items = nch * ntiles;
        auto ld_part = [&](const char* base, uint32_t o) {
            return __hip_atomic_load(reinterpret_cast<const float*>(base + o * 4u), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
        };
        for (int g0 = 0; g0 < items; g0 += kGroup) {
            float vc[kGroup][kRpt], vr[kGroup][kRpt], zg[kGroup][kRpt];
            uint32_t orow[kGroup][kRpt];
            bool okrow[kGroup][kRpt];
            // 1. every load of the group: column-major sums of column j0 + r,
            //    row i0 + tx (to transpose), and the row-major sums (and z)
            //    of row i0 + r, column j0 + tx
#pragma unroll
            for (int g = 0; g < kGroup; ++g) {
                const int it = g0 + g;
                const bool have = it < items;                     // uniform
                const int c = have ? it / ntiles : 0, tile_id = have ? it % ntiles : 0;
                const uint32_t off = static_cast<uint32_t>((b * a.dim + dfirst + c) * a.L);
                const int i0 = (tile_id / tiles_w) * kTr, j0 = (tile_id % tiles_w) * kTr;
#pragma unroll
                for (int q = 0; q < kRpt; ++q) {
                    const int r = ty + q * (kThreads / kTr);
                    const bool okc = have && i0 + tx < H && j0 + r < Wd;
                    vc[g][q] = okc ? ld_part(p1, off + static_cast<uint32_t>((j0 + r) * H + i0 + tx)) : 0.f;
                    okrow[g][q] = have && i0 + r < H && j0 + tx < Wd;
                    orow[g][q] = off + static_cast<uint32_t>((i0 + r) * Wd + j0 + tx);
                    vr[g][q] = okrow[g][q] ? ld_part(p0, orow[g][q]) : 0.f;
                    zg[g][q] = 1.f;
                    if (GATE && okrow[g][q])
                        zg[g][q] = from_raw<T>(ld_raw(reinterpret_cast<const T*>(zb + orow[g][q] * kEs), 0));
                }
            }
            // 2. the column-major tiles into LDS, transposed on the way out
#pragma unroll
            for (int g = 0; g < kGroup; ++g)
#pragma unroll
                for (int q = 0; q < kRpt; ++q) tr[g][ty + q * (kThreads / kTr)][tx] = vc[g][q];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
            // 3. y = (row-major pair + column-major pair) * gate
#pragma unroll
            for (int g = 0; g < kGroup; ++g)
#pragma unroll
                for (int q = 0; q < kRpt; ++q) {
                    if (!okrow[g][q]) continue;
                    float v = vr[g][q] + tr[g][tx][ty + q * (kThreads / kTr)];
                    if (GATE) v *= silu_f(zg[g][q]);
                    st(reinterpret_cast<T*>(yb + orow[g][q] * kEs), 0, v);
                }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        }
    }
}

// ---------------------------------------------------------------- gradient
// Reverse-mode gradient of the Vim scan (vim_scan_bidir_grad). Same row
// layout as rowscan_kernel (one recurrence per 16-lane row, lane n = state
// n, CH channels x {forward, backward} per workgroup: 24 when that still
// gives every CU a workgroup, else 8) with the blocks taken in reverse
// order. Per block:
//   * the states h_t of the block's 16 steps are recomputed from the state
//     stored at the block's start by the forward pass (rowscan_kernel with
//     CKPT), keeping h_t and e_t = exp(delta_t A_n) in registers;
//   * the adjoint runs backwards over the 16 steps,
//       lam_t = gs_t C_t + e_{t+1} lam_{t+1},  gs = dy * silu(z),
//     carrying e_{t+1} lam_{t+1} from step to step and across blocks;
//   * per step and state: q = (lam e_t) h_{t-1}, dA += q delta_t,
//     dC_t = gs_t h_t, dB_t = lam_t delta_t u_t; the sums over states
//     R_w = sum_n lam B_t and R_v = sum_n q A_n are row transpose
//     reductions (lane j ends with step j's sums), giving
//       du_t = delta_t R_w + gs_t D,  ddelta_t = R_v + u_t R_w,
//       ddelta_raw = ddelta_t * softplus'(x_t) = ddelta_t * sigmoid(x_t);
//   * du and ddelta of the two directions merge through fp32 partial sums
//     as the forward merge does (blocks above F hold first visits, below F
//     second visits, block F is mixed);
//   * dB and dC are shared by every channel: each lane holds its state's
//     contributions for the block's 16 steps. A 32-lane swap sums the wave's
//     two rows of the same direction (dB lands in the low half of the wave,
//     dC in the high half), LDS sums the workgroup's waves, and the workgroup
//     stores its 1024 block sums (dB|dC x side x step x state) as one
//     contiguous 4 KB chunk. grad_bc_reduce_kernel then sums the chunks over
//     the workgroups in a fixed order, so no atomics are involved and dB and
//     dC repeat bit for bit. dA, dD and dt_bias are summed per row, stored
//     per batch row, and summed over the batch rows by the same kernel, in
//     order, so they repeat bit for bit as well.
using vs::kBcChunk;               // floats per workgroup and block: [dB|dC][side][step][n]

struct GradArgs {
    const void *u, *delta, *z, *B, *C, *dy;
    const float *A, *Dskip, *dt_bias;
    const float* s;         // merged ungated forward output (fp32)
    const float* ckpt;      // state at each block start, per row
    float *pdu, *pdd;       // fp32 partial sums of du and ddelta_raw
    void *du, *ddelta, *dz;
    float *bc_part;         // [batch][group][block][kBcChunk] dB/dC chunks
    float *pstat;           // per batch row: dA, dD, dt_bias sums (kernel-wide strides)
    int64_t dim, L;
    int dstate, nblk;
};

__device__ __forceinline__ float sigmoid_f(float x) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

// Lanes 0-31 return a[l] + a[l + 32]; lanes 32-63 return b[l - 32] + b[l]
// (one v_permlane32_swap, which exchanges the upper half of a with the lower
// half of b, and one add).
__device__ __forceinline__ float swap32_sum(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename T, bool GATE, bool SOFTPLUS, int CH>
__global__ __launch_bounds__(CH * 2 * kRowLanes) __attribute__((amdgpu_waves_per_eu(3)))
void rowgrad_kernel(const GradArgs a) {
    // CH channels x {forward, backward} rows per workgroup, two channels per wave
    constexpr int kChPerWg = CH;
    constexpr int kWaves = CH / 2;
    static_assert(CH % 4 == 0, "whole waves, and at least the 256 staging threads");
    __shared__ __attribute__((aligned(16))) float tile[2][2][2][kRowLanes][kTilePad];
    // per wave and lane: the 16 steps' dB|dC sums after the 32-lane swap, as
    // four float4 (steps 4q..4q+3) stored lane after lane, so that the
    // writes and the summing reads are both contiguous across lanes; two
    // buffers, so that a block's sums are reduced while the waves go on to
    // the next block (one barrier per block)
    __shared__ float4 red[2][kWaves][4][kWaveLanes];

    const int tid = threadIdx.x;
    const int lane = tid & (kWaveLanes - 1);
    const int row_in_wg = tid >> 4;
    const int n = lane & (kRowLanes - 1);
    const int dir = row_in_wg & 1;
    const int ch = row_in_wg >> 1;
    uint32_t cg, bb;
    xcd_block(cg, bb);
    const int64_t b = bb;
    const int64_t d0 = static_cast<int64_t>(cg) * kChPerWg + ch;
    const bool active = d0 < a.dim;
    const int64_t d = active ? d0 : 0;
    const int L = static_cast<int>(a.L);
    const int nblk = a.nblk;
    const bool rev = dir == 1;
    const int64_t prow = dir * a.dim + d;
    const bool n_ok = active && n < a.dstate;
    const float An = n_ok ? a.A[prow * a.dstate + n] : 0.f;
    const float A2 = An * kLog2e;
    const float Dk = (active && a.Dskip) ? a.Dskip[prow] : 0.f;
    const float bias = (active && a.dt_bias) ? a.dt_bias[prow] : 0.f;

    constexpr uint32_t kEs = sizeof(T);
    const uint32_t rowoff = static_cast<uint32_t>((b * a.dim + d) * a.L);
    const char* __restrict__ ub = static_cast<const char*>(a.u);
    const char* __restrict__ db = static_cast<const char*>(a.delta);
    const char* __restrict__ zb = static_cast<const char*>(a.z);
    const char* __restrict__ gb = static_cast<const char*>(a.dy);
    const char* __restrict__ sb = reinterpret_cast<const char*>(a.s);
    auto act_at = [&](const char* base, int p) {
        return ld_raw(reinterpret_cast<const T*>(base + (rowoff + static_cast<uint32_t>(p)) * kEs), 0);
    };
    auto f32_at = [&](const char* base, int p) {
        return reinterpret_cast<const float*>(base + (rowoff + static_cast<uint32_t>(p)) * 4u);
    };
    auto out_at = [&](void* base, int p) {
        return reinterpret_cast<T*>(static_cast<char*>(base) + (rowoff + static_cast<uint32_t>(p)) * kEs);
    };
    float* const pdu = a.pdu + rowoff;
    float* const pdd = a.pdd + rowoff;
    const float* const ck_row =
        a.ckpt + ((static_cast<size_t>(b * a.dim + d) * 2 + dir) * nblk) * kRowLanes;

    // ---- B/C staging (as rowscan_kernel: side 0 reads token t, side 1 L-1-t),
    // by the first 256 threads (whole waves; the other waves load nothing):
    // thread (sn, slot) moves state sn of step slot
    constexpr int kStage = 4;
    const bool stager = __builtin_amdgcn_readfirstlane(tid >> 6) < kThreads / kWaveLanes;
    const int sn = (tid >> 4) & (kRowLanes - 1), slot = tid & 15;
    const bool sn_ok = sn < a.dstate;
    const uint32_t bc_row = static_cast<uint32_t>((b * a.dstate + (sn_ok ? sn : 0)) * a.L);
    const char* __restrict__ Bb = static_cast<const char*>(a.B);
    const char* __restrict__ Cb = static_cast<const char*>(a.C);
    auto stage_load = [&](int blk, uint32_t (&sr)[kStage]) VS_INLINE {
        if (!stager) return;
        const int t = blk * kBlockTok + slot;
        const int tc = t < L ? t : L - 1;
#pragma unroll
        for (int r = 0; r < kStage; ++r) {
            const uint32_t off = (bc_row + static_cast<uint32_t>((r >> 1) ? L - 1 - tc : tc)) * kEs;
            sr[r] = ld_raw(reinterpret_cast<const T*>(((r & 1) ? Cb : Bb) + off), 0);
        }
    };
    const int st_col = sn_ok ? slot : kRowLanes;
    auto stage_store = [&](int buf, const uint32_t (&sr)[kStage]) VS_INLINE {
        if (stager) {
#pragma unroll
            for (int r = 0; r < kStage; ++r)
                tile[buf][r >> 1][r & 1][sn][st_col] = from_raw<T>(sr[r]);
        }
    };
    if (stager && !sn_ok) {
#pragma unroll
        for (int r = 0; r < kStage; ++r) {
            tile[0][r >> 1][r & 1][sn][slot] = 0.f;
            tile[1][r >> 1][r & 1][sn][slot] = 0.f;
        }
    }
    // after the swap, lane l of a wave holds which = l / 32 (dB, dC),
    // side = (l / 16) & 1 (the rows' direction) and state l % 16; the chunk
    // is [which][side][step][state]
    float* const bc_chunks = a.bc_part + static_cast<size_t>(b * gridDim.x + cg) * nblk * kBcChunk;
    // the first 256 threads sum and store the chunk: thread (q = tid / 64,
    // l = tid % 64) steps 4q..4q+3 of wave lane l, at chunk floats
    // 256 (l / 16) + 16 step + l % 16; the others get an out-of-range offset
    const int red_q = (tid >> 6) & 3;
    const int chunk_off = stager ? ((lane >> 4) * 256 + red_q * 64 + (lane & 15)) * 4 : kBcChunk * 4;

    auto tok_pos = [&](int blk) {
        const int t = blk * kBlockTok + n;
        const int tc = t < L ? t : L - 1;
        return rev ? L - 1 - tc : tc;
    };
    const int Fstep = (L - 1) / (2 * kBlockTok);
    struct Tok { uint32_t u, dl, z, g; float s, h0; int p; };
    auto tok_load = [&](int blk, Tok& k) VS_INLINE {
        const int p = tok_pos(blk);
        k.p = p;
        const float h0 = ck_row[blk * kRowLanes + n];            // state at the block's start
        k.h0 = active ? h0 : 0.f;
        k.u = act_at(ub, p);
        k.dl = act_at(db, p);
        k.g = act_at(gb, p);
        if (GATE) {
            k.z = act_at(zb, p);
            k.s = *f32_at(sb, p);
        }
    };

    // Per-token outputs go through buffer descriptors that cover the wave's
    // two channels; a lane with nothing to store gets the first offset past
    // that range, which the hardware drops. The loop bodies then have no
    // divergent branches around memory operations, so the waits the compiler
    // inserts for the prefetched loads do not also wait for these stores.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);      // uniform per wave
    const int64_t wave_d0 = static_cast<int64_t>(cg) * kChPerWg + 2 * wave;
    const int64_t wave_ch = a.dim - wave_d0 < 0 ? 0 : (a.dim - wave_d0 > 2 ? 2 : a.dim - wave_d0);
    const size_t wave_el = static_cast<size_t>(b * a.dim + (wave_ch > 0 ? wave_d0 : 0)) * a.L;
    const uint32_t wave_n = static_cast<uint32_t>(wave_ch * a.L);
    auto rsrc = [&](void* base, uint32_t es) {
        return __builtin_amdgcn_make_buffer_rsrc(static_cast<char*>(base) + wave_el * es, 0,
                                                 static_cast<int>(wave_n * es), 0x00020000);
    };
    const auto r_du = rsrc(a.du, kEs), r_dd = rsrc(a.ddelta, kEs);
    const auto r_pdu = rsrc(a.pdu, 4), r_pdd = rsrc(a.pdd, 4);
    const auto r_dz = GATE ? rsrc(a.dz, kEs) : r_du;
    const uint32_t row_el = static_cast<uint32_t>((d - (wave_ch > 0 ? wave_d0 : 0)) * a.L);
    auto bst = [&](__amdgpu_buffer_rsrc_t r, uint32_t es, bool on, int p, float v) {
        const int off = static_cast<int>(on ? (row_el + static_cast<uint32_t>(p)) * es : wave_n * es);
        if (es == 4)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v)),
                                                  r, off, 0, 0);
    };

    uint32_t sr[kStage];
    const int last = nblk - 1;
    stage_load(last, sr);
    stage_store(last & 1, sr);
    Tok tA{}, tB{};
    tok_load(last, tA);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

    // Blocks above F hold every token's first visit (its partial du, ddelta
    // go to pdu, pdd, and dz is written there), blocks below F the second
    // (partial added, du and ddelta written); block F mixes both.
    constexpr int kFirst = 0, kMixed = 1, kSecond = 2;
    float lamE = 0.f, dA_acc = 0.f, dD_acc = 0.f, dbias_acc = 0.f;
    auto step = [&](auto phase, const int blk, Tok& cur, Tok& nxt) VS_INLINE {
        constexpr int PH = decltype(phase)::value;
        const int buf = blk & 1;
        const int p = cur.p;
        const bool ok = active && blk * kBlockTok + n < L;
        // partial sums of the other direction's first visits
        float part_du = 0.f, part_dd = 0.f;
        if (PH == kSecond) {
            part_du = __hip_atomic_load(pdu + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            part_dd = __hip_atomic_load(pdd + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const int nb = blk > 0 ? blk - 1 : 0;
        stage_load(nb, sr);
        tok_load(nb, nxt);

        // this lane's step (slot n) quantities
        const float cu = from_raw<T>(cur.u);
        const float x = from_raw<T>(cur.dl) + bias;
        const float sp = SOFTPLUS ? softplus_f(x) : x;
        const float dlt = ok ? sp : 0.f;
        const float du_ = dlt * cu;
        const float g = from_raw<T>(cur.g);
        float gs = g;
        if (GATE) {
            const float zz = from_raw<T>(cur.z);
            const float sg = sigmoid_f(zz);
            gs = g * zz * sg;
            // dz at the token's first visit
            const float dzv = g * cur.s * sg * fmaf(zz, 1.f - sg, 1.f);
            if (PH == kFirst) {
                bst(r_dz, kEs, ok, p, dzv);
            } else if (PH == kMixed) {
                const int t_self = blk * kBlockTok + n;
                const int blk_other = (L - 1 - t_self) / kBlockTok;
                if (ok && (blk > blk_other || (blk == blk_other && dir == 0)))
                    st(out_at(a.dz, p), 0, dzv);
            }
        }
        gs = ok ? gs : 0.f;
        // second copies of the broadcast sources, opaque to the compiler, so
        // that each broadcast has one use and folds into it as a DPP operand
        // (one shared broadcast would cost a separate v_mov_b32_dpp)
        float du2 = du_, gs2 = gs;
        asm volatile("" : "+v"(du2), "+v"(gs2));

        const float4* Bt = reinterpret_cast<const float4*>(&tile[buf][dir][0][n][0]);
        const float4* Ct = reinterpret_cast<const float4*>(&tile[buf][dir][1][n][0]);
        float Bv[16], Cv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 bq = Bt[q], cq = Ct[q];
            Bv[4 * q] = bq.x; Bv[4 * q + 1] = bq.y; Bv[4 * q + 2] = bq.z; Bv[4 * q + 3] = bq.w;
            Cv[4 * q] = cq.x; Cv[4 * q + 1] = cq.y; Cv[4 * q + 2] = cq.z; Cv[4 * q + 3] = cq.w;
        }
        // recompute the block's states from the stored start state
        const float h_in = cur.h0;
        float hs[16], es[16];
        {
            float h = h_in;
            Unroll<16>::run([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                es[i] = __builtin_amdgcn_exp2f(row_bcast<i>(dlt) * A2);
                h = fmaf(es[i], h, row_bcast<i>(du_) * Bv[i]);
                hs[i] = h;
            });
        }
        // adjoint, backwards over the block's steps: lam_i = e_{i+1} lam_{i+1}
        // + gs_i C_i, where lamE = e_{i+1} lam_{i+1} comes from the step
        // before (zero past the sequence's end)
        float wv[16], vv[16], sbc[16];
        Unroll<16>::run([&](auto ic) {
            constexpr int i = 15 - decltype(ic)::value;
            const float lam = row_bcast_fmac<i, i == 15>(lamE, gs, Cv[i]);
            lamE = lam * es[i];
            const float hprev = i > 0 ? hs[i > 0 ? i - 1 : 0] : h_in;
            const float q = lamE * hprev;
            dA_acc = row_bcast_fmac<i, i == 15>(dA_acc, dlt, q);
            wv[i] = lam * Bv[i];
            vv[i] = q * An;
            sbc[i] = swap32_sum(row_bcast<i>(du2) * lam, row_bcast<i>(gs2) * hs[i]);
        });
        const float Rw = row_transpose_sum(wv, lane);
        const float Rv = row_transpose_sum(vv, lane);
        const float du_tok = fmaf(dlt, Rw, gs * Dk);
        const float ddl = fmaf(cu, Rw, Rv);
        const float dx = SOFTPLUS ? ddl * sigmoid_f(x) : ddl;
        if (ok) {
            dbias_acc += dx;
            dD_acc = fmaf(gs, cu, dD_acc);
        }
        // merge the two directions' du and ddelta_raw for this step's token
        if (PH == kFirst) {
            bst(r_pdu, 4, ok, p, du_tok);
            bst(r_pdd, 4, ok, p, dx);
        } else if (PH == kSecond) {
            bst(r_du, kEs, ok, p, du_tok + part_du);
            bst(r_dd, kEs, ok, p, dx + part_dd);
        } else {
            const int t_self = blk * kBlockTok + n;
            const int blk_other = (L - 1 - t_self) / kBlockTok;
            const bool first = blk > blk_other || (blk == blk_other && dir == 0);
            if (ok && first) {
                __hip_atomic_store(pdu + p, du_tok, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(pdd + p, dx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
            if (ok && !first) {
                const float odu = __hip_atomic_load(pdu + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const float odd = __hip_atomic_load(pdd + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                st(out_at(a.du, p), 0, du_tok + odu);
                st(out_at(a.ddelta, p), 0, dx + odd);
            }
        }

        // stage the next block's B/C (that buffer was last read before the
        // previous barrier), write this block's dB/dC sums, and after the
        // barrier sum the waves' sums into the block's chunk. The next block
        // writes the other sum buffer, whose reduction finished before this
        // barrier, so one barrier per block covers both.
        stage_store(buf ^ 1, sr);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            red[blk & 1][tid >> 6][q][lane] = make_float4(sbc[4 * q], sbc[4 * q + 1], sbc[4 * q + 2], sbc[4 * q + 3]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        if (stager) {
            const int rb = blk & 1;
            float4 acc = red[rb][0][red_q][lane];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) {
                const float4 v = red[rb][w][red_q][lane];
                acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
            }
            const auto rc = __builtin_amdgcn_make_buffer_rsrc(bc_chunks + static_cast<size_t>(blk) * kBcChunk,
                                                              0, kBcChunk * 4, 0x00020000);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc.x), rc, chunk_off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc.y), rc, chunk_off + 64, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc.z), rc, chunk_off + 128, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc.w), rc, chunk_off + 192, 0, 0);
        }
    };

    // Each phase is its own loop with the same memory operations on every
    // trip; everything in flight is drained between the phases.
    // the issue priority steps down at each quarter of the blocks, as in
    // rowscan_kernel, so that the workgroups sharing a CU finish together
    int blk = last;
    const int g1 = last - nblk / 4, g3 = last - (3 * nblk) / 4;
    __builtin_amdgcn_s_setprio(3);
    __builtin_amdgcn_s_waitcnt(0);
    for (; blk > Fstep; --blk) {
        if (blk == g1) __builtin_amdgcn_s_setprio(2);
        step(std::integral_constant<int, kFirst>{}, blk, tA, tB);
        tA = tB;
    }
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_s_waitcnt(0);
    step(std::integral_constant<int, kMixed>{}, blk, tA, tB);
    tA = tB;
    __builtin_amdgcn_s_waitcnt(0);
    for (--blk; blk >= 0; --blk) {
        if (blk == g3) __builtin_amdgcn_s_setprio(0);
        step(std::integral_constant<int, kSecond>{}, blk, tA, tB);
        tA = tB;
    }

    // per-row sums: dA (lane n), dD and dt_bias (summed over the row's lanes),
    // stored for this batch row; grad_bc_reduce_kernel sums the batch rows
    float* const ps = a.pstat + static_cast<size_t>(b) * 2 * a.dim * (a.dstate + 2);
    if (n_ok) ps[prow * a.dstate + n] = dA_acc;
    float sD = dD_acc, sb2 = dbias_acc;
    sD += dpp<0x4e>(sD); sb2 += dpp<0x4e>(sb2);              // quad_perm [2,3,0,1]
    sD += dpp<0xb1>(sD); sb2 += dpp<0xb1>(sb2);              // quad_perm [1,0,3,2]
    sD += dpp<0x114>(sD); sb2 += dpp<0x114>(sb2);            // row_shr:4 (lane 15: + lane 11)
    sD += dpp<0x118>(sD); sb2 += dpp<0x118>(sb2);            // row_shr:8 (lane 15: + lane 7)
    if (active && n == 15) {
        ps[2 * a.dim * a.dstate + prow] = sD;
        ps[2 * a.dim * (a.dstate + 1) + prow] = sb2;
    }
}

// dB and dC from the gradient kernel's chunks: the sum over the workgroups of
// side 0 at step t = token t and side 1 at step t = token L-1-t. A thread
// takes four consecutive states of one token (16-byte loads), a workgroup
// 64 tokens; the workgroups of the gradient are added in a fixed order. The
// workgroups past the token range of batch row 0 sum dA, dD and dt_bias over
// the batch rows, in order, one thread per output.
constexpr int kRedTok = kThreads / 4;       // tokens per reduction workgroup
__global__ __launch_bounds__(kThreads) void grad_bc_reduce_kernel(
        const float* __restrict__ part, float* __restrict__ dB, float* __restrict__ dC, int64_t L,
        int dstate, int nblk, int ngroups, const float* __restrict__ pstat, float* __restrict__ dA,
        float* __restrict__ dD, float* __restrict__ dbias, int64_t dim, int batch) {
    const int ntb = static_cast<int>((L + kRedTok - 1) / kRedTok);
    if (static_cast<int>(blockIdx.x) >= ntb) {
        const int64_t np = 2 * dim * (dstate + 2);
        const int64_t k = static_cast<int64_t>(blockIdx.x - ntb) * kThreads + threadIdx.x;
        if (blockIdx.y != 0 || k >= np) return;
        float sum = 0.f;
        for (int b = 0; b < batch; ++b) sum += pstat[static_cast<size_t>(b) * np + k];
        const int64_t na = 2 * dim * dstate;
        if (k < na) dA[k] = sum;
        else if (k < na + 2 * dim) dD[k - na] = sum;
        else dbias[k - na - 2 * dim] = sum;
        return;
    }
    const int q = threadIdx.x & 3;              // states 4q .. 4q + 3
    const int64_t b = blockIdx.y;
    const int64_t tok = static_cast<int64_t>(blockIdx.x) * kRedTok + (threadIdx.x >> 2);
    if (tok >= L || 4 * q >= dstate) return;
    const int64_t t1 = L - 1 - tok;
    // [which][side][step][n]: side 0 for the forward direction, 1 for the
    // backward one; every (side, step) row of a chunk is read by the
    // threads whose token it holds
    const size_t o0 = static_cast<size_t>(tok / kBlockTok) * kBcChunk +
                      static_cast<size_t>(tok % kBlockTok) * kRowLanes + 4 * q;
    const size_t o1 = static_cast<size_t>(t1 / kBlockTok) * kBcChunk +
                      static_cast<size_t>(kBlockTok + t1 % kBlockTok) * kRowLanes + 4 * q;
    constexpr size_t kC = kBcChunk / 2;
    const size_t gstride = static_cast<size_t>(nblk) * kBcChunk;
    const float* c = part + static_cast<size_t>(b) * ngroups * gstride;
    float4 sB = make_float4(0.f, 0.f, 0.f, 0.f), sC = sB;
    auto add2 = [](float4& s, const float4 x, const float4 y) {
        s.x += x.x + y.x; s.y += x.y + y.y; s.z += x.z + y.z; s.w += x.w + y.w;
    };
    for (int g = 0; g < ngroups; ++g, c += gstride) {
        add2(sB, *reinterpret_cast<const float4*>(c + o0), *reinterpret_cast<const float4*>(c + o1));
        add2(sC, *reinterpret_cast<const float4*>(c + o0 + kC), *reinterpret_cast<const float4*>(c + o1 + kC));
    }
    const float vb[4] = {sB.x, sB.y, sB.z, sB.w}, vc[4] = {sC.x, sC.y, sC.z, sC.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (4 * q + k >= dstate) break;
        const size_t o = static_cast<size_t>(b * dstate + 4 * q + k) * static_cast<size_t>(L) +
                         static_cast<size_t>(tok);
        dB[o] = vb[k];
        dC[o] = vc[k];
    }
}

// Transpose u and delta of every (batch, channel) from the row-major H x W
// grid to column-major order (entry j*H + i = grid element (i, j)), in 32 x
// 32 tiles through LDS so that reads and writes are both contiguous.
template <typename T>
__global__ __launch_bounds__(kThreads) void grid_transpose_kernel(
    const T* __restrict__ u, const T* __restrict__ dl, T* __restrict__ uT, T* __restrict__ dT,
    int H, int W, int64_t nrows) {
    // u's and delta's tile of the same (batch, channel) row in one
    // workgroup: all 8 loads of a thread are issued before the barrier
    __shared__ T tr[2][kTr][kTr + 1];
    const int tiles_w = (W + kTr - 1) / kTr;
    const int i0 = (blockIdx.x / tiles_w) * kTr, j0 = (blockIdx.x % tiles_w) * kTr;
    const int tx = threadIdx.x & (kTr - 1), ty = threadIdx.x / kTr;
    const int64_t L = static_cast<int64_t>(H) * W;
    for (int64_t row = blockIdx.y; row < nrows; row += gridDim.y) {
        const int64_t base = row * L;
#pragma unroll
        for (int r = ty; r < kTr; r += kThreads / kTr) {
            const int i = i0 + r, j = j0 + tx;
            if (i < H && j < W) {
                tr[0][r][tx] = u[base + static_cast<int64_t>(i) * W + j];
                tr[1][r][tx] = dl[base + static_cast<int64_t>(i) * W + j];
            }
        }
        __syncthreads();
#pragma unroll
        for (int r = ty; r < kTr; r += kThreads / kTr) {
            const int j = j0 + r, i = i0 + tx;
            if (i < H && j < W) {
                uT[base + static_cast<int64_t>(j) * H + i] = tr[0][tx][r];
                dT[base + static_cast<int64_t>(j) * H + i] = tr[1][tx][r];
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- host side
// Argument records and their validation live in host.cpp (vs_internal.h);
// this file launches the kernels for calls that passed it.
using vs::Call;
using vs::GradCall;
using vs::fail;

template <typename T>
void launch_chunked(const Call& c, dim3 grid, dim3 blk, hipStream_t st, const ScanArgs& a) {
    constexpr int V = kModeVim;
    if (c.z && c.softplus)
        hipLaunchKernelGGL((rowscan_kernel<T, V, true, true, false, false, false, true>), grid, blk, 0, st, a);
    else if (c.z)
        hipLaunchKernelGGL((rowscan_kernel<T, V, true, false, false, false, false, true>), grid, blk, 0, st, a);
    else if (c.softplus)
        hipLaunchKernelGGL((rowscan_kernel<T, V, false, true, false, false, false, true>), grid, blk, 0, st, a);
    else
        hipLaunchKernelGGL((rowscan_kernel<T, V, false, false, false, false, false, true>), grid, blk, 0, st, a);
}

// the Vim scan with its partial sums in LDS (lds bytes of dynamic LDS),
// chunked or not
template <typename T, bool CHUNK>
void launch_vim_plds(const Call& c, dim3 grid, dim3 blk, hipStream_t st, const ScanArgs& a, size_t lds) {
    constexpr int V = kModeVim;
    const unsigned sh = static_cast<unsigned>(lds);
    if (c.z && c.softplus)
        hipLaunchKernelGGL((rowscan_kernel<T, V, true, true, false, false, false, CHUNK, false, true>), grid, blk, sh, st, a);
    else if (c.z)
        hipLaunchKernelGGL((rowscan_kernel<T, V, true, false, false, false, false, CHUNK, false, true>), grid, blk, sh, st, a);
    else if (c.softplus)
        hipLaunchKernelGGL((rowscan_kernel<T, V, false, true, false, false, false, CHUNK, false, true>), grid, blk, sh, st, a);
    else
        hipLaunchKernelGGL((rowscan_kernel<T, V, false, false, false, false, false, CHUNK, false, true>), grid, blk, sh, st, a);
}

// Chunks per sequence for a plain Vim scan. Unchunked, the launch has
// batch * ceil(dim / 8) workgroups of 4 waves; below 2 waves per SIMD (1,024
// SIMDs) the chip is under-filled and the sequential length sets the time, so
// the sequence is cut into chunks until the grid reaches about 3 waves per
// SIMD, and into at most 3: each chunk first rescans its prefix or suffix
// (measured: Vim-B 2048^2, 1.5 waves per SIMD unchunked, 0.766 ms, 2 chunks
// 0.694 ms, 3 chunks 0.873 ms; Vim-Ti 224^2, 0.19 waves per SIMD, 11.1,
// 11.7, 10.2 and 10.9 us per step for 1 to 4 chunks). Never more chunks
// than 32-token tiles.
int chunk_count(const Call& c) {
    const int64_t ntile = (c.L + vs::kTileTok - 1) / vs::kTileTok;
    int64_t k = c.chunks;
    if (k == 0) {
        const int64_t waves = c.batch * ((c.dim + 7) / 8) * 4;
        const int64_t simds = vs::kNumCUs * 4;
        k = waves >= 2 * simds ? 1 : (3 * simds) / waves;
        k = k < 1 ? 1 : (k > 3 ? 3 : k);
    }
    // at most one chunk per tile, and grid.y = batch * chunks within 65535
    const int64_t kmax = 65535 / c.batch;
    k = k < ntile ? k : ntile;
    return static_cast<int>(k < kmax ? k : kmax);
}

template <typename T, int MODE, bool CONV, bool ZOH>
void launch_scan(const Call& c, dim3 grid, dim3 blk, hipStream_t st, const ScanArgs& a) {
    if (c.z && c.softplus)
        hipLaunchKernelGGL((rowscan_kernel<T, MODE, true, true, CONV, false, ZOH>), grid, blk, 0, st, a);
    else if (c.z)
        hipLaunchKernelGGL((rowscan_kernel<T, MODE, true, false, CONV, false, ZOH>), grid, blk, 0, st, a);
    else if (c.softplus)
        hipLaunchKernelGGL((rowscan_kernel<T, MODE, false, true, CONV, false, ZOH>), grid, blk, 0, st, a);
    else
        hipLaunchKernelGGL((rowscan_kernel<T, MODE, false, false, CONV, false, ZOH>), grid, blk, 0, st, a);
}

// the cross-scan with its u and delta grids staged in LDS (lds bytes of
// dynamic LDS)
template <typename T, bool ZOH>
void launch_cross4_lds(const Call& c, dim3 grid, dim3 blk, hipStream_t st, const ScanArgs& a, size_t lds) {
    constexpr int M = kModeCross4;
    const unsigned sh = static_cast<unsigned>(lds);
    if (c.z && c.softplus)
        hipLaunchKernelGGL((rowscan_kernel<T, M, true, true, false, false, ZOH, false, true>), grid, blk, sh, st, a);
    else if (c.z)
        hipLaunchKernelGGL((rowscan_kernel<T, M, true, false, false, false, ZOH, false, true>), grid, blk, sh, st, a);
    else if (c.softplus)
        hipLaunchKernelGGL((rowscan_kernel<T, M, false, true, false, false, ZOH, false, true>), grid, blk, sh, st, a);
    else
        hipLaunchKernelGGL((rowscan_kernel<T, M, false, false, false, false, ZOH, false, true>), grid, blk, sh, st, a);
}

template <typename T, int MODE>
int launch_t(const Call& c) {
    ScanArgs a{};
    a.u = c.u; a.delta = c.delta; a.z = c.z; a.B = c.B; a.C = c.C;
    a.A = c.A; a.Dskip = c.Dskip; a.dt_bias = c.dt_bias; a.y = c.y;
    a.conv_w = c.conv_w; a.conv_b = c.conv_b;
    a.dir_off = c.per_dir ? static_cast<uint32_t>(c.batch * c.dim * c.L) : 0u;
    a.bc_per_dir = c.per_dir ? 1 : 0;
    // merge buffers: fp32 y doubles as the first one; the cross-scan's second
    // pair always uses the workspace (after the first buffer if y is bf16)
    float* ws = static_cast<float*>(c.ws);
    const int64_t elems = c.batch * c.dim * c.L;
    a.partial = c.dtype == VS_F32 ? static_cast<float*>(c.y) : ws;
    a.partial2 = nullptr;
    a.uT = a.deltaT = nullptr;
    const bool grid_lds = MODE == kModeCross4 && vs::cross4_grid_in_lds(c.L, c.dtype);
    if (MODE == kModeCross4) {
        // workspace: [bf16 only: pair-0 sums][pair-1 sums][u^T][delta^T],
        // the transposed copies only for grids too large for LDS
        a.partial2 = c.dtype == VS_F32 ? ws : ws + elems;
        if (!grid_lds) {
            T* act = reinterpret_cast<T*>(a.partial2 + elems);
            a.uT = act;
            a.deltaT = act + elems;
        }
    }
    a.dim = c.dim; a.L = c.L; a.H = c.H; a.W = c.W;
    a.dstate = static_cast<int>(c.dstate);
    a.softplus = c.softplus ? 1 : 0;
    a.reverse = c.reverse ? 1 : 0;
    a.nblk = static_cast<int>((c.L + kBlockTok - 1) / kBlockTok);
    constexpr int kChPerWg = MODE == kModeVim ? 8 : (MODE == kModeCross4 ? 4 : 16);
    dim3 grid(static_cast<unsigned>((c.dim + kChPerWg - 1) / kChPerWg),
              static_cast<unsigned>(c.batch));
    hipStream_t st = static_cast<hipStream_t>(c.stream);
    const dim3 blk(kThreads);
    if (MODE == kModeCross4 && !grid_lds) {
        const int64_t rows = c.batch * c.dim;
        const unsigned tiles = static_cast<unsigned>(((c.H + kTr - 1) / kTr) * ((c.W + kTr - 1) / kTr));
        const unsigned gy = static_cast<unsigned>(rows < 65535 ? rows : 65535);
        hipLaunchKernelGGL((grid_transpose_kernel<T>), dim3(tiles, gy, 1), blk, 0, st,
                           static_cast<const T*>(c.u), static_cast<const T*>(c.delta),
                           const_cast<T*>(static_cast<const T*>(a.uT)),
                           const_cast<T*>(static_cast<const T*>(a.deltaT)), c.H, c.W, rows);
    }
    if constexpr (MODE == kModeVim) {
        // the plain scan takes chunks when the grid under-fills the chip
        const bool plain = !c.conv_w && !c.zoh && !c.per_dir;
        const int nchunk = plain ? chunk_count(c) : 1;
        // the longest chunk (whole 32-token tiles but the last) and whether
        // its workgroup's partial sums fit in LDS
        const int64_t ntile = (c.L + vs::kTileTok - 1) / vs::kTileTok;
        const int64_t lc_tiled = (ntile + nchunk - 1) / nchunk * vs::kTileTok;
        const int64_t Lc = lc_tiled < c.L ? lc_tiled : c.L;
        const size_t plds = static_cast<size_t>(vs::vim_partial_lds_bytes(Lc));
        const bool use_plds = !c.conv_w && !c.zoh && plds <= static_cast<size_t>(vs::kPartLdsBytes);
        if (nchunk > 1) {
            ScanArgs ac = a;
            ac.nchunk = nchunk;
            const dim3 cgrid(grid.x, grid.y * static_cast<unsigned>(nchunk));
            if (use_plds) launch_vim_plds<T, true>(c, cgrid, blk, st, ac, plds);
            else launch_chunked<T>(c, cgrid, blk, st, ac);
        } else if (use_plds) {
            launch_vim_plds<T, false>(c, grid, blk, st, a, plds);
        } else if (c.conv_w) {
            if (c.zoh) launch_scan<T, MODE, true, true>(c, grid, blk, st, a);
            else launch_scan<T, MODE, true, false>(c, grid, blk, st, a);
        } else if (c.zoh) {
            launch_scan<T, MODE, false, true>(c, grid, blk, st, a);
        } else {
            launch_scan<T, MODE, false, false>(c, grid, blk, st, a);
        }
    } else if (grid_lds) {
        const size_t lds = static_cast<size_t>(2 * vs::kCrossChPerWg * c.L) * sizeof(T);
        if (c.zoh) launch_cross4_lds<T, true>(c, grid, blk, st, a, lds);
        else launch_cross4_lds<T, false>(c, grid, blk, st, a, lds);
    } else if (c.zoh) {
        launch_scan<T, MODE, false, true>(c, grid, blk, st, a);
    } else {
        launch_scan<T, MODE, false, false>(c, grid, blk, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(VS_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return VS_OK;
}

// ---- gradient of the Vim scan (workspace layout: vs::grad_ws_bytes)
using vs::grad_channels;
using vs::grad_ws_bytes;
using vs::grad_saved_bytes;
using vs::grad_rest_bytes;

template <typename T, int CH>
void launch_rowgrad(bool gate, bool softplus, dim3 grid, hipStream_t st, const GradArgs& r) {
    const dim3 blk(CH * 2 * kRowLanes);
    if (gate && softplus)
        hipLaunchKernelGGL((rowgrad_kernel<T, true, true, CH>), grid, blk, 0, st, r);
    else if (gate)
        hipLaunchKernelGGL((rowgrad_kernel<T, true, false, CH>), grid, blk, 0, st, r);
    else if (softplus)
        hipLaunchKernelGGL((rowgrad_kernel<T, false, true, CH>), grid, blk, 0, st, r);
    else
        hipLaunchKernelGGL((rowgrad_kernel<T, false, false, CH>), grid, blk, 0, st, r);
}

// The checkpointing forward pass (rowscan_kernel with CKPT): the merged
// ungated output s (fp32) and the state at every block start into the saved
// buffer, and the gated y as well when y is given.
template <typename T>
void launch_ckpt_forward(const void* u, const void* delta, const void* z, const void* B, const void* C,
                         const float* A, const float* Dskip, const float* dt_bias, int softplus, void* y,
                         float* sbuf, float* ckpt, int64_t batch, int64_t dim, int64_t dstate, int64_t L,
                         hipStream_t st) {
    ScanArgs a{};
    a.u = u; a.delta = delta; a.z = z; a.B = B; a.C = C;
    a.A = A; a.Dskip = Dskip; a.dt_bias = dt_bias; a.y = y;
    a.partial = sbuf; a.ckpt = ckpt;
    a.dim = dim; a.L = L; a.dstate = static_cast<int>(dstate);
    a.softplus = softplus; a.nblk = static_cast<int>((L + kBlockTok - 1) / kBlockTok);
    constexpr int kFwdCh = 8;      // rowscan_kernel (Vim): 8 channels x 2 directions per workgroup
    const dim3 fgrid(static_cast<unsigned>((dim + kFwdCh - 1) / kFwdCh), static_cast<unsigned>(batch));
    const dim3 blk(kThreads);
    if (z && softplus)
        hipLaunchKernelGGL((rowscan_kernel<T, kModeVim, true, true, false, true>), fgrid, blk, 0, st, a);
    else if (z)
        hipLaunchKernelGGL((rowscan_kernel<T, kModeVim, true, false, false, true>), fgrid, blk, 0, st, a);
    else if (softplus)
        hipLaunchKernelGGL((rowscan_kernel<T, kModeVim, false, true, false, true>), fgrid, blk, 0, st, a);
    else
        hipLaunchKernelGGL((rowscan_kernel<T, kModeVim, false, false, false, true>), fgrid, blk, 0, st, a);
}

// vim_scan_bidir_fwd_saved: y and the saved buffer (c.ws)
template <typename T>
int launch_fwd_saved(const Call& c) {
    size_t so[2];
    grad_saved_bytes(c.batch, c.dim, c.L, so);
    char* sv = static_cast<char*>(c.ws);
    launch_ckpt_forward<T>(c.u, c.delta, c.z, c.B, c.C, c.A, c.Dskip, c.dt_bias, c.softplus, c.y,
                           reinterpret_cast<float*>(sv + so[0]), reinterpret_cast<float*>(sv + so[1]),
                           c.batch, c.dim, c.dstate, c.L, static_cast<hipStream_t>(c.stream));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(VS_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return VS_OK;
}

template <typename T>
int launch_grad(const GradCall& g) {
    // s and the checkpoints come from the saved buffer of a saving forward
    // call, or from the first part of the workspace, filled here
    size_t so[2], ro[4];
    const size_t saved_size = grad_saved_bytes(g.batch, g.dim, g.L, so);
    grad_rest_bytes(g.batch, g.dim, g.L, ro);
    char* ws = static_cast<char*>(g.ws);
    // the kernels only read s and the checkpoints of a saved buffer
    char* sv = g.saved ? const_cast<char*>(static_cast<const char*>(g.saved)) : ws;
    char* rest = g.saved ? ws : ws + saved_size;
    float* sbuf = reinterpret_cast<float*>(sv + so[0]);
    float* ckpt = reinterpret_cast<float*>(sv + so[1]);
    hipStream_t st = static_cast<hipStream_t>(g.stream);
    const dim3 blk(kThreads);
    const int ch = grad_channels(g.batch, g.dim);
    const unsigned groups = static_cast<unsigned>((g.dim + ch - 1) / ch);
    const dim3 grid(groups, static_cast<unsigned>(g.batch));
    const int nblk = static_cast<int>((g.L + kBlockTok - 1) / kBlockTok);
    // 1. forward pass: merged ungated output (fp32) and the states at every
    //    block start (not needed after a saving forward call)
    if (!g.saved)
        launch_ckpt_forward<T>(g.u, g.delta, nullptr, g.B, g.C, g.A, g.Dskip, g.dt_bias, g.softplus, nullptr,
                               sbuf, ckpt, g.batch, g.dim, g.dstate, g.L, st);
    // 2. reverse pass
    GradArgs r{};
    r.u = g.u; r.delta = g.delta; r.z = g.z; r.B = g.B; r.C = g.C; r.dy = g.dy;
    r.A = g.A; r.Dskip = g.Dskip; r.dt_bias = g.dt_bias;
    r.s = sbuf; r.ckpt = ckpt;
    r.pdu = reinterpret_cast<float*>(rest + ro[0]);
    r.pdd = reinterpret_cast<float*>(rest + ro[1]);
    r.du = g.du; r.ddelta = g.ddelta; r.dz = g.dz;
    r.bc_part = reinterpret_cast<float*>(rest + ro[2]);
    r.pstat = reinterpret_cast<float*>(rest + ro[3]);
    r.dim = g.dim; r.L = g.L; r.dstate = static_cast<int>(g.dstate); r.nblk = nblk;
    if (ch == 24)
        launch_rowgrad<T, 24>(g.z != nullptr, g.softplus != 0, grid, st, r);
    else
        launch_rowgrad<T, 8>(g.z != nullptr, g.softplus != 0, grid, st, r);
    // 3. dB and dC; dA, dD and dt_bias
    const int64_t pblocks = (2 * g.dim * (g.dstate + 2) + kThreads - 1) / kThreads;
    const int64_t ntb = (g.L + kRedTok - 1) / kRedTok;
    hipLaunchKernelGGL(grad_bc_reduce_kernel,
                       dim3(static_cast<unsigned>(ntb + pblocks), static_cast<unsigned>(g.batch)), blk, 0, st,
                       r.bc_part, g.dB, g.dC, g.L, static_cast<int>(g.dstate), nblk, static_cast<int>(groups),
                       r.pstat, g.dA, g.dD, g.dbias, g.dim, static_cast<int>(g.batch));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(VS_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return VS_OK;
}

// launches a call that passed vs::prepare
int dispatch(const Call& c) {
    const bool bf = c.dtype == VS_BF16;
    switch (c.mode) {
    case kMode1D: return bf ? launch_t<uint16_t, kMode1D>(c) : launch_t<float, kMode1D>(c);
    case kModeVim: return bf ? launch_t<uint16_t, kModeVim>(c) : launch_t<float, kModeVim>(c);
    default: return bf ? launch_t<uint16_t, kModeCross4>(c) : launch_t<float, kModeCross4>(c);
    }
}

int run(Call c) {
    const int rc = vs::prepare(c);
    return rc != VS_OK ? rc : dispatch(c);
}

// ---- the merge buffer of vim_scan_bidir_noalloc: a static device array
// (each GPU that loads the library holds its own copy until the process
// ends). Host code never uses the array's name as an address: the device
// address is looked up once per device with that device current and kept.
constexpr size_t kScratchFloats = VS_NOALLOC_MAX_ELEMS;
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices];

int scratch_on_current_device(float** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(VS_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(VS_ERR_UNSUPPORTED, "device index above 63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(VS_ERR_HIP, std::string("hipGetSymbolAddress: ") + hipGetErrorString(e));
        g_scratch_ptr[dev] = static_cast<float*>(p);
    }
    *out = g_scratch_ptr[dev];
    return VS_OK;
}

}  // namespace

// ---------------------------------------------------------------- C ABI
extern "C" {

int vim_scan_bidir(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                   const void* u, const void* delta, const void* z, const void* B,
                   const void* C, const float* A, const float* Dskip, const float* dt_bias,
                   int delta_softplus, void* y, void* workspace, size_t workspace_bytes,
                   void* stream) {
    Call c{kModeVim, batch, dim, dstate, seqlen, 0, 0, dtype, 0, u, delta, z, B, C,
           A, Dskip, dt_bias, delta_softplus, y, workspace, workspace_bytes, stream};
    return run(c);
}

int vim_scan_bidir_chunked(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                           const void* u, const void* delta, const void* z, const void* B,
                           const void* C, const float* A, const float* Dskip, const float* dt_bias,
                           int delta_softplus, int chunks, void* y, void* workspace,
                           size_t workspace_bytes, void* stream) {
    Call c{kModeVim, batch, dim, dstate, seqlen, 0, 0, dtype, 0, u, delta, z, B, C,
           A, Dskip, dt_bias, delta_softplus, y, workspace, workspace_bytes, stream};
    c.chunks = chunks;
    return run(c);
}

int vim_scan_bidir_noalloc(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                           const void* u, const void* delta, const void* z, const void* B,
                           const void* C, const float* A, const float* Dskip, const float* dt_bias,
                           int delta_softplus, void* y, void* stream) {
    Call c{kModeVim, batch, dim, dstate, seqlen, 0, 0, dtype, 0, u, delta, z, B, C,
           A, Dskip, dt_bias, delta_softplus, y, nullptr, kScratchFloats * sizeof(float), stream};
    c.ws_internal = true;
    int rc = vs::prepare(c);        // sizes first: nothing below runs for a refused call
    if (rc != VS_OK) return rc;
    float* buf = nullptr;
    rc = scratch_on_current_device(&buf);
    if (rc != VS_OK) return rc;
    c.ws = buf;
    return dispatch(c);
}

int vim_scan_bidir_dirs(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                        const void* u, const void* delta, const void* z, const void* B,
                        const void* C, const float* A, const float* Dskip, const float* dt_bias,
                        int delta_softplus, void* y, void* workspace, size_t workspace_bytes,
                        void* stream) {
    Call c{kModeVim, batch, dim, dstate, seqlen, 0, 0, dtype, 0, u, delta, z, B, C,
           A, Dskip, dt_bias, delta_softplus, y, workspace, workspace_bytes, stream};
    c.per_dir = true;
    return run(c);
}
int vim_scan_bidir_conv(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                        const void* x, const float* conv_w, const float* conv_b,
                        const void* delta, const void* z, const void* B, const void* C,
                        const float* A, const float* Dskip, const float* dt_bias,
                        int delta_softplus, void* y, void* workspace, size_t workspace_bytes,
                        void* stream) {
    Call c{kModeVim, batch, dim, dstate, seqlen, 0, 0, dtype, 0, x, delta, z, B, C,
           A, Dskip, dt_bias, delta_softplus, y, workspace, workspace_bytes, stream};
    c.conv = true;
    c.conv_w = conv_w;
    c.conv_b = conv_b;
    return run(c);
}

int vim_scan_bidir_grad(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                        const void* u, const void* delta, const void* z, const void* B,
                        const void* C, const float* A, const float* Dskip, const float* dt_bias,
                        int delta_softplus, const void* dy, void* du, void* ddelta, void* dz,
                        float* dB, float* dC, float* dA, float* dD, float* ddt_bias,
                        void* workspace, size_t workspace_bytes, void* stream) {
    vs::clear_error();
    GradCall g{batch, dim, dstate, seqlen, dtype, u, delta, z, B, C, A, Dskip, dt_bias,
               delta_softplus, dy, du, ddelta, dz, dB, dC, dA, dD, ddt_bias,
               workspace, workspace_bytes, stream};
    const int rc = vs::validate_grad(g);
    if (rc != VS_OK) return rc;
    return dtype == VS_BF16 ? launch_grad<uint16_t>(g) : launch_grad<float>(g);
}

int vim_scan_bidir_fwd_saved(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                             const void* u, const void* delta, const void* z, const void* B,
                             const void* C, const float* A, const float* Dskip, const float* dt_bias,
                             int delta_softplus, void* y, void* saved, size_t saved_bytes, void* stream) {
    Call c{kModeVim, batch, dim, dstate, seqlen, 0, 0, dtype, 0, u, delta, z, B, C,
           A, Dskip, dt_bias, delta_softplus, y, saved, saved_bytes, stream};
    c.saved_fwd = true;
    const int rc = vs::prepare(c);
    if (rc != VS_OK) return rc;
    return dtype == VS_BF16 ? launch_fwd_saved<uint16_t>(c) : launch_fwd_saved<float>(c);
}

int vim_scan_bidir_grad_saved(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                              const void* u, const void* delta, const void* z, const void* B,
                              const void* C, const float* A, const float* Dskip, const float* dt_bias,
                              int delta_softplus, const void* saved, size_t saved_bytes, const void* dy,
                              void* du, void* ddelta, void* dz, float* dB, float* dC, float* dA, float* dD,
                              float* ddt_bias, void* workspace, size_t workspace_bytes, void* stream) {
    vs::clear_error();
    if (!saved) return fail(VS_ERR_NULL, "saved must not be NULL");
    GradCall g{batch, dim, dstate, seqlen, dtype, u, delta, z, B, C, A, Dskip, dt_bias,
               delta_softplus, dy, du, ddelta, dz, dB, dC, dA, dD, ddt_bias,
               workspace, workspace_bytes, stream};
    g.saved = saved;
    g.saved_bytes = saved_bytes;
    const int rc = vs::validate_grad(g);
    if (rc != VS_OK) return rc;
    return dtype == VS_BF16 ? launch_grad<uint16_t>(g) : launch_grad<float>(g);
}

int vmamba_cross_scan4(int64_t batch, int64_t dim, int64_t dstate, int64_t H, int64_t W,
                       int dtype, const void* u, const void* delta, const void* z,
                       const void* B, const void* C, const float* A, const float* Dskip,
                       const float* dt_bias, int delta_softplus, void* y, void* workspace,
                       size_t workspace_bytes, void* stream) {
    vs::clear_error();
    if (!vs::grid_ok(H, W)) return fail(VS_ERR_SHAPE, "H and W must be in 1..2^20");
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

}  // extern "C"
