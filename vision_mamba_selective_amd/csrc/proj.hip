// proj.hip -- the linear maps around the scan, on gfx950 matrix cores.
//
// "Vision Mamba Guide: Efficient Bidirectional SSM & VMamba", section
// "1. PyTorch Implementation of the Bidirectional Vision Mamba Block":
// SimpleSelectiveSSM's x_proj (Linear(d_model, 2 d_state + 1), no bias)
// produces B, C and a one-wide dt; dt_proj (Linear(1, d_model)) widens dt
// per channel inside the softplus; the block's out_proj (Linear(d_model,
// d_model)) maps the fused output before the residual is added. In the
// channel-major layout [batch][features][L] of the scan, nn.Linear's
// out = in W^T + b is, for every batch row b and token t,
//     out[b][m][t] = sum_k W[m][k] in[b][k][t] (+ bias[m]) (+ residual[b][m][t]).
//
// proj_gemm_kernel computes one batch row's Out[M][L] = W[M][K] X[K][L] in
// BM x BN tiles with v_mfma_f32_32x32x16_bf16 (bf16 operands, fp32
// accumulation), which takes 8 consecutive k of one row of W (A) and of one
// column of X (B) per lane. Per slice of K (128 deep, 64 for out_proj's
// short-sequence tile), W's rows are copied to LDS as they are (k
// contiguous), and X's rows too (token contiguous), 16 bytes per load: X
// rows start at any 2-byte boundary (L is odd), which the target's
// unaligned global access handles.
// The B fragments come out of LDS
// with ds_read_b64_tr_b16, which transposes 4 x 16 blocks of b16 within each
// 16-lane group: a lane reading 4 tokens of one k row contributes element i
// to lane i of its group, so every lane receives 4 consecutive k of its own
// token. The next slice is loaded into registers while the matrix cores
// work on the current one (two slices ahead measured slower: the second
// register set costs more occupancy than the latency it hides). The
// workgroup's 2 x WN waves each own (BM/2) x (BN/WN) of the tile: out_proj
// takes 128 x 128 tiles in 8 waves from 1,024 tokens on (128 x 64 in 4
// below), x_proj 64 x 64 tiles in 4. out_proj's epilogue stages the tile
// through LDS, so that the residual is read and the result written in whole
// rows. In the last tile of a row, which passes the sequence end, the one
// 8-token chunk per row that straddles the end is read and written entry by
// entry, and the chunks past it are not touched; these tiles are dispatched
// first.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "vimscan.h"
#include "vs_internal.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kThreads = 256;
constexpr int64_t kWideTileMinL = 1024;    // out_proj: 128-token tiles from this length on
constexpr int kXPad = 16;               // X slice rows: BN + 16 bf16, 160 bytes for BN = 64,
                                        // which puts the 4 rows x 2 token halves that a
                                        // transposing read touches per 32 lanes on
                                        // distinct banks

enum { kEpiOut = 0, kEpiXproj = 1 };

struct ProjArgs {
    const uint16_t* W;     // [M][K] bf16
    const uint16_t* X;     // [batch][K][L] bf16
    const float* bias;     // [M] fp32 or null
    const uint16_t* res;   // [batch][M][L] bf16 or null
    uint16_t* out;         // kEpiOut: [batch][M][L] bf16
    uint16_t* B;           // kEpiXproj: rows 0..N-1 -> B [batch][N][L]
    uint16_t* C;           //            rows N..2N-1 -> C [batch][N][L]
    float* dt;             //            row 2N -> dt [batch][L] (fp32)
    int M, K, N, L;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));   // round to nearest even
}

typedef __attribute__((ext_vector_type(4))) short v4s;

// BK: K per LDS slice. W's slice rows are BK + 8 bf16 (16 bytes of padding),
// which keeps the fragment reads of 16 lanes on distinct banks.
// WN: waves across the tile's tokens (2 across its rows), 2 x WN waves of
// 64 lanes in the workgroup, each owning (BM / 2) x (BN / WN) of the tile.
template <int BM, int BN, int BK, int EPI, bool WVEC, int WN>
__global__ __launch_bounds__(128 * WN) void proj_gemm_kernel(const ProjArgs a) {
    constexpr int kWgThreads = 128 * WN;
    static_assert(BM % 64 == 0 && BN % (32 * WN) == 0, "2 x WN waves of 32 x 32 MFMA tiles");
    static_assert(BK % 16 == 0, "whole MFMA k steps per slice");
    constexpr int kBK = BK;
    constexpr int kRow = BK + 8;
    constexpr int TM = BM / 64, TN = BN / (32 * WN);
    // X slice: kBK rows of BN tokens, 16-byte chunks of 8 tokens
    // rows of BN + 16 bf16 for BN = 64 (40 dwords mod 64 banks) and BN + 32
    // for BN = 128 (16 dwords mod 64: the 4 rows of a transposing read, 16
    // dwords each with both token halves, fill the 64 banks once)
    constexpr int kXRow = BN + (BN >= 128 ? 32 : kXPad);
    constexpr int kXChunks = kBK * BN / 8;
    static_assert(kXChunks % kWgThreads == 0, "whole chunks per thread");
    constexpr int kXcpt = kXChunks / kWgThreads;
    // W slice: 16-byte chunks (WVEC) or single elements
    constexpr int kChunks = BM * kBK / 8;
    constexpr int kChunkPT = (kChunks + kWgThreads - 1) / kWgThreads;
    constexpr int kElemPT = BM * kBK / kWgThreads;

    // the operand slices; after the K loop the same memory holds the output
    // tile (bf16, rows of BN + 8), staged so that residual reads and result
    // writes move whole rows of the tile
    constexpr int kOutRow = BN + 8;
    constexpr int kOps = BM * kRow + kBK * kXRow;
    constexpr int kSmem = kOps > BM * kOutRow ? kOps : BM * kOutRow;
    __shared__ __attribute__((aligned(16))) uint16_t smem[kSmem];
    __shared__ float sBias[BM];
    uint16_t (*sA)[kRow] = reinterpret_cast<uint16_t (*)[kRow]>(smem);
    uint16_t (*sX)[kXRow] = reinterpret_cast<uint16_t (*)[kXRow]>(smem + BM * kRow);
    uint16_t (*sT)[kOutRow] = reinterpret_cast<uint16_t (*)[kOutRow]>(smem);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    // Workgroups are dealt to the 8 XCDs (each with its own L2) round-robin by
    // linear id; renumber them so that each XCD runs one contiguous range of
    // tiles. Neighbouring M tiles read the same X columns, which then stay
    // in that XCD's L2 instead of being fetched from HBM once per tile.
    uint32_t mt, nt, bt;
    {
        constexpr uint32_t kXcds = 8;
        const uint32_t gx = gridDim.x, gy = gridDim.y;
        const uint32_t G = gx * gy * gridDim.z;
        const uint32_t lin = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
        const uint32_t x = lin % kXcds, k = lin / kXcds, q = G / kXcds, r = G % kXcds;
        const uint32_t v = x * q + (x < r ? x : r) + k;
        mt = v % gx;
        // token tiles in reverse order: a row's last tile, which passes the
        // sequence end and reads its straddling chunks entry by entry, starts
        // first instead of forming the kernel's tail
        nt = gy - 1 - (v / gx) % gy;
        bt = v / (gx * gy);
    }
    const int m0 = mt * BM, n0 = nt * BN;
    const int64_t b = bt;
    const int M = a.M, K = a.K, L = a.L;
    const uint16_t* __restrict__ Xb = a.X + b * static_cast<int64_t>(K) * L;

    // the tile's tokens all lie inside the sequence (uniform per workgroup).
    // Else each 8-token chunk is read whole if it lies inside, entry by
    // entry (clamped) if it straddles the end, and not at all past it: tokens
    // past L feed only output columns that are never stored.
    const bool xwhole = n0 + BN <= L;
    auto load_chunk = [&](const uint16_t* src, int t0) -> uint4 {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (xwhole || t0 + 8 <= L) {
            __builtin_memcpy(&v, src + t0, 16);
        } else if (t0 < L) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int u0 = t0 + 2 * e, u1 = u0 + 1;
                w[e] = uint32_t(src[u0 < L ? u0 : L - 1]) | (uint32_t(src[u1 < L ? u1 : L - 1]) << 16);
            }
            v = make_uint4(w[0], w[1], w[2], w[3]);
        }
        return v;
    };

    uint4 wreg[WVEC ? kChunkPT : 1];
    uint16_t wel[WVEC ? 1 : kElemPT];
    uint4 xreg[kXcpt];
    auto load_slice = [&](int k0) {
        if (WVEC) {
#pragma unroll
            for (int i = 0; i < kChunkPT; ++i) {
                const int c = tid + i * kWgThreads;
                const int r = c / (kBK / 8), kc = (c % (kBK / 8)) * 8;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (c < kChunks && m0 + r < M && k0 + kc < K)
                    v = *reinterpret_cast<const uint4*>(a.W + static_cast<int64_t>(m0 + r) * K + k0 + kc);
                wreg[i] = v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kElemPT; ++i) {
                const int e = tid + i * kWgThreads;
                const int r = e / kBK, kk = e % kBK;
                wel[i] = (m0 + r < M && k0 + kk < K) ? a.W[static_cast<int64_t>(m0 + r) * K + k0 + kk] : 0;
            }
        }
#pragma unroll
        for (int i = 0; i < kXcpt; ++i) {
            const int c = tid + i * kWgThreads;
            const int r = c / (BN / 8), nc = (c % (BN / 8)) * 8;
            // rows past K: any finite value (W is zero there)
            const uint16_t* src = Xb + static_cast<int64_t>(k0 + r < K ? k0 + r : K - 1) * L;
            xreg[i] = load_chunk(src, n0 + nc);
        }
    };
    auto store_slice = [&]() {
        if (WVEC) {
#pragma unroll
            for (int i = 0; i < kChunkPT; ++i) {
                const int c = tid + i * kWgThreads;
                if (c < kChunks)
                    *reinterpret_cast<uint4*>(&sA[c / (kBK / 8)][(c % (kBK / 8)) * 8]) = wreg[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < kElemPT; ++i) {
                const int e = tid + i * kWgThreads;
                sA[e / kBK][e % kBK] = wel[i];
            }
        }
#pragma unroll
        for (int i = 0; i < kXcpt; ++i) {
            const int c = tid + i * kWgThreads;
            *reinterpret_cast<uint4*>(&sX[c / (BN / 8)][(c % (BN / 8)) * 8]) = xreg[i];
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    if (EPI == kEpiOut && tid < BM)
        sBias[tid] = (a.bias && m0 + tid < M) ? a.bias[m0 + tid] : 0.f;
    const int fr = lane & 31, fk = 8 * (lane >> 5);     // fragment row / column, k offset
    // transposing reads of X: lane 4e + q of a 16-lane group reads 4 tokens
    // (4q ..) of k row e of its group's 4 x 16 block; group g covers k rows
    // 8 (g / 2) .. and tokens 16 (g % 2) ..
    const int tg = lane >> 4, tp = lane & 15;
    const int tk = 8 * (tg >> 1) + (tp >> 2), tn = 16 * (tg & 1) + 4 * (tp & 3);
    load_slice(0);
    for (int k0 = 0; k0 < K; k0 += kBK) {
        store_slice();
        __syncthreads();
        if (k0 + kBK < K) load_slice(k0 + kBK);
#pragma unroll
        for (int ks = 0; ks < kBK; ks += 16) {
            bf16x8 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                fa[i] = *reinterpret_cast<const bf16x8*>(&sA[wm * (BM / 2) + i * 32 + fr][ks + fk]);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int nb = wn * (BN / WN) + j * 32 + tn;
                const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4s*)(&sX[ks + tk][nb]));
                const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4s*)(&sX[ks + tk + 4][nb]));
                const __attribute__((ext_vector_type(8))) short v8 = {lo[0], lo[1], lo[2], lo[3],
                                                                     hi[0], hi[1], hi[2], hi[3]};
                fb[j] = __builtin_bit_cast(bf16x8, v8);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // accumulator r of lane l: row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
    if (EPI == kEpiOut) {
        // 1. the residual tile into LDS, 16 bytes (8 tokens of a row) per
        //    load; in the last tile of a row, a chunk that straddles the end
        //    entry by entry, clamped (rows and columns past the matrix: any
        //    valid element or zero, never stored)
        constexpr int kOutChunks = BM * BN / 8;
        static_assert(kOutChunks % kWgThreads == 0, "whole chunks per thread");
        constexpr int kOcpt = kOutChunks / kWgThreads;
        if (a.res) {
#pragma unroll
            for (int q = 0; q < kOcpt; ++q) {
                const int c = tid + q * kWgThreads;
                const int row = c / (BN / 8), nc = (c % (BN / 8)) * 8;
                const int64_t mcl = m0 + row < M ? m0 + row : M - 1;
                const uint16_t* src = a.res + (b * M + mcl) * static_cast<int64_t>(L);
                *reinterpret_cast<uint4*>(&sT[row][nc]) = load_chunk(src, n0 + nc);
            }
        }
        __syncthreads();
        // 2. each lane finishes its own elements in place: acc + bias + residual
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int cn = wn * (BN / WN) + j * 32 + fr;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int cm = wm * (BM / 2) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    float v = acc[i][j][r] + sBias[cm];
                    if (a.res) v += bf16_to_f32(sT[cm][cn]);
                    sT[cm][cn] = f32_to_bf16(v);
                }
            }
        __syncthreads();
        // 3. the tile out, 16 bytes per store (a chunk that straddles the
        //    sequence end entry by entry; chunks past it are not stored)
#pragma unroll
        for (int q = 0; q < kOcpt; ++q) {
            const int c = tid + q * kWgThreads;
            const int row = c / (BN / 8), nc = (c % (BN / 8)) * 8;
            if (m0 + row >= M) continue;
            uint16_t* dst = a.out + (b * M + m0 + row) * static_cast<int64_t>(L) + n0 + nc;
            const uint4 v = *reinterpret_cast<const uint4*>(&sT[row][nc]);
            if (xwhole || n0 + nc + 8 <= L) {
                __builtin_memcpy(dst, &v, 16);
            } else if (n0 + nc < L) {
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (n0 + nc + e < L) dst[e] = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
            }
        }
    } else {
        // x_proj: rows 0..N-1 -> B, N..2N-1 -> C (bf16), row 2N -> dt (fp32)
        const int N = a.N;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = n0 + wn * (BN / WN) + j * 32 + fr;
                if (n >= L) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + wm * (BM / 2) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (m >= M) continue;
                    const float v = acc[i][j][r];
                    if (m < N)
                        a.B[(b * N + m) * static_cast<int64_t>(L) + n] = f32_to_bf16(v);
                    else if (m < 2 * N)
                        a.C[(b * N + (m - N)) * static_cast<int64_t>(L) + n] = f32_to_bf16(v);
                    else
                        a.dt[b * L + n] = v;
                }
            }
    }
}

// dt_proj without its bias: delta[b][d][t] = w[d] dt[b][t], in bf16. A thread
// takes kDtTok consecutive tokens of kDtCh channels: it reads their dt once
// and writes 16 bytes per channel (rows start at any 2-byte boundary, which
// the target's unaligned global access handles; the last chunk of a row,
// past the sequence end, is written entry by entry).
constexpr int kDtTok = 8, kDtCh = 8;
__global__ __launch_bounds__(kThreads) void dt_proj_kernel(const float* __restrict__ dt,
                                                           const float* __restrict__ w,
                                                           uint16_t* __restrict__ delta, int dim,
                                                           int L) {
    const int t0 = (blockIdx.x * kThreads + threadIdx.x) * kDtTok;
    if (t0 >= L) return;
    const int64_t b = blockIdx.z;
    const int d0 = blockIdx.y * kDtCh;
    const float* src = dt + b * L + t0;
    const bool whole = t0 + kDtTok <= L;
    float v[kDtTok];
    if (whole) {
        __builtin_memcpy(v, src, sizeof(v));
    } else {
#pragma unroll
        for (int i = 0; i < kDtTok; ++i) v[i] = t0 + i < L ? src[i] : 0.f;
    }
#pragma unroll
    for (int c = 0; c < kDtCh; ++c) {
        const int d = d0 + c;
        if (d >= dim) break;
        const float wd = w[d];
        uint32_t pk[kDtTok / 2];
#pragma unroll
        for (int i = 0; i < kDtTok / 2; ++i)
            pk[i] = uint32_t(f32_to_bf16(wd * v[2 * i])) | (uint32_t(f32_to_bf16(wd * v[2 * i + 1])) << 16);
        uint16_t* dst = delta + (b * dim + d) * static_cast<int64_t>(L) + t0;
        if (whole) {
            __builtin_memcpy(dst, pk, sizeof(pk));
        } else {
#pragma unroll
            for (int e = 0; e < kDtTok; ++e)
                if (t0 + e < L) dst[e] = static_cast<uint16_t>(pk[e >> 1] >> (16 * (e & 1)));
        }
    }
}

using vs::fail;

template <int BM, int BN, int BK, int EPI, int WN>
int launch(const ProjArgs& a, int64_t batch, hipStream_t st) {
    const int64_t tiles_l = (static_cast<int64_t>(a.L) + BN - 1) / BN;
    if (tiles_l > 65535)
        return fail(VS_ERR_UNSUPPORTED, "sequence too long for the projection grid");
    const dim3 grid(static_cast<unsigned>((a.M + BM - 1) / BM), static_cast<unsigned>(tiles_l),
                    static_cast<unsigned>(batch));
    const bool wvec = a.K % 8 == 0 && vs::aligned(a.W, 16);
    if (wvec)
        hipLaunchKernelGGL((proj_gemm_kernel<BM, BN, BK, EPI, true, WN>), grid, dim3(128 * WN), 0, st, a);
    else
        hipLaunchKernelGGL((proj_gemm_kernel<BM, BN, BK, EPI, false, WN>), grid, dim3(128 * WN), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(VS_ERR_HIP, hipGetErrorString(e));
    return VS_OK;
}

}  // namespace

extern "C" {

int vim_x_proj(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
               const void* u, const void* W, void* B, void* C, float* dt, void* stream) {
    const int rc = vs::validate_x_proj(batch, dim, dstate, seqlen, dtype, u, W, B, C, dt);
    if (rc != VS_OK) return rc;
    const int64_t M = 2 * dstate + 1;
    ProjArgs a{};
    a.W = static_cast<const uint16_t*>(W);
    a.X = static_cast<const uint16_t*>(u);
    a.B = static_cast<uint16_t*>(B);
    a.C = static_cast<uint16_t*>(C);
    a.dt = dt;
    a.M = static_cast<int>(M); a.K = static_cast<int>(dim);
    a.N = static_cast<int>(dstate); a.L = static_cast<int>(seqlen);
    // 128-deep slices: same output bits as 64-deep ones, 14.4 against 15.6 us
    // at 197 tokens (batch 64), 19.8 against 20.1 us at 4,097 (batch 8)
    return launch<64, 64, 128, kEpiXproj, 2>(a, batch, static_cast<hipStream_t>(stream));
}

int vim_dt_proj(int64_t batch, int64_t dim, int64_t seqlen, int dtype, const float* dt,
                const float* w, void* delta, void* stream) {
    const int rc = vs::validate_dt_proj(batch, dim, seqlen, dtype, dt, w, delta);
    if (rc != VS_OK) return rc;
    const int64_t per_wg = static_cast<int64_t>(kThreads) * kDtTok;
    const dim3 grid(static_cast<unsigned>((seqlen + per_wg - 1) / per_wg),
                    static_cast<unsigned>((dim + kDtCh - 1) / kDtCh), static_cast<unsigned>(batch));
    hipLaunchKernelGGL(dt_proj_kernel, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), dt, w,
                       static_cast<uint16_t*>(delta), static_cast<int>(dim), static_cast<int>(seqlen));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(VS_ERR_HIP, hipGetErrorString(e));
    return VS_OK;
}

int vim_out_proj(int64_t batch, int64_t dim_in, int64_t dim_out, int64_t seqlen, int dtype,
                 const void* y, const void* W, const float* bias, const void* residual, void* out,
                 void* stream) {
    const int rc = vs::validate_out_proj(batch, dim_in, dim_out, seqlen, dtype, y, W, bias, residual, out);
    if (rc != VS_OK) return rc;
    ProjArgs a{};
    a.W = static_cast<const uint16_t*>(W);
    a.X = static_cast<const uint16_t*>(y);
    a.bias = bias;
    a.res = static_cast<const uint16_t*>(residual);
    a.out = static_cast<uint16_t*>(out);
    a.M = static_cast<int>(dim_out); a.K = static_cast<int>(dim_in); a.L = static_cast<int>(seqlen);
    // Long sequences take 128 x 128 tiles in eight waves (each 64 x 32, as in
    // the 128 x 64 tiles of four waves) and 128-deep K slices: W is read once
    // per 128 tokens instead of 64, a workgroup has 64 KB of operands in
    // flight per slice, and four times the matrix work sits between a
    // slice's barriers; same output bits. Short sequences keep 128 x 64
    // tiles: at 197 tokens (batch 64) the wider tile took 68 against 54 us.
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (seqlen >= kWideTileMinL) return launch<128, 128, 128, kEpiOut, 4>(a, batch, st);
    return launch<128, 64, 64, kEpiOut, 2>(a, batch, st);
}

}  // extern "C"
