// fp4q_gemm.hip -- MXFP4 GEMM on the gfx950 scaled matrix cores.
//
// C (M x N) = A_hat (M x K) * B_hat^T, where A and B are MXFP4 matrices in the
// layout the quantize kernels write: row-major E2M1 codes two per byte (element
// 2j in the low nibble) and one E8M0 scale byte per 32 consecutive elements of
// a row.  For an activation-times-weight product A holds the activations
// (tokens x in-features) and B the weights (out-features x in-features).
//
// The hot loop is v_mfma_scale_f32_16x16x128_f8f6f4 with both operands in E2M1
// (format 4) and a per-lane E8M0 scale for each.  For that instruction lane l
// supplies row l % 16 of its 16 x 128 operand over the 32-element K block
// l / 16, as 16 bytes of packed codes, plus that block's scale byte; lane l
// receives C[4 (l / 16) + i][l % 16], i = 0..3.  A lane's operand is therefore
// exactly 16 contiguous bytes of one row of the stored codes: the matrices are
// consumed as the quantizer wrote them, without repacking.
//
// Tiling: a workgroup of 4 waves computes a 128 x 128 tile of C; wave (wm, wn)
// a 64 x 64 sub-tile as 4 x 4 MFMAs.  K advances 128 at a time through
// double-buffered LDS stages (codes 128 rows x 64 bytes plus 4 scale bytes per
// row, for A and for B): the next stage's global loads are issued before the
// current stage's MFMAs and written to LDS after them.  All global accesses are
// range-checked buffer operations, so tiles that overhang M, N or K read zeros
// (code +0, which contributes nothing) and drop their stores.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "fp4q_launch.h"

namespace fp4q {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

constexpr int kWave = 64;
constexpr int kThreads = 256;
constexpr int BM = 128, BN = 128, BK = 128;   // workgroup tile and K step
constexpr int kRowBytes = BK / 2;             // packed codes per tile row per stage
constexpr int kLdsRow = kRowBytes + 16;       // padded LDS row (spreads the banks)
constexpr int kFmtE2M1 = 4;                   // MFMA operand format: FP4 E2M1
constexpr int kDropped = (int)0x80000000;     // an offset past every buffer range
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

struct GParams {
    const uint8_t* a_codes;
    const uint8_t* a_scales;
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    int64_t M, N, K;
    void* c;
    int ct;  // 0 bf16, 1 f32
};

// One stage of global data held in registers between its load and its LDS
// write: each thread moves 2 x 16 bytes of codes of A and of B, and one row's
// 4 scale bytes (of A for threads below 128, of B above).
struct Stage {
    u32x4_t a[2], b[2];
    uint32_t sc;
};

// The workgroup's operand windows: buffer resources based at its first row of
// A and of B (so every offset stays within one 128-row slab), sized to the
// rows that exist.
struct Tiles {
    Rsrc a, b, sa, sb;
};

// Thread t moves rows t / 4 and 64 + t / 4, 16-byte segment t % 4 of the
// stage's 64 code bytes per row; segments past K read zeros (code +0).
// Threads t < 128 also move the 4 scale bytes of A's row t, t >= 128 those of
// B's row t - 128 (as byte loads: a row's scale bytes need not be aligned).
__device__ __forceinline__ void load_stage(Stage& s, const GParams& p, const Tiles& w,
                                           int64_t k0) {
    const int t = threadIdx.x;
    const int seg = t & 3;
    const bool kin = k0 + seg * 32 < p.K;  // the segment's 32 elements are inside K
    const int rowb = (int)(p.K / 2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = (t >> 2) + h * 64;
        const int o = kin ? r * rowb + (int)(k0 / 2) + seg * 16 : kDropped;
        s.a[h] = __builtin_amdgcn_raw_buffer_load_b128(w.a, o, 0, 0);
        s.b[h] = __builtin_amdgcn_raw_buffer_load_b128(w.b, o, 0, 0);
    }
    const int srow = (int)(p.K / 32);
    const int r = t & 127;
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int off = (k0 / 32 + q) < srow ? r * srow + (int)(k0 / 32) + q : kDropped;
        const uint32_t byte = t >= 128 ? __builtin_amdgcn_raw_buffer_load_b8(w.sb, off, 0, 0)
                                       : __builtin_amdgcn_raw_buffer_load_b8(w.sa, off, 0, 0);
        word |= byte << (8 * q);
    }
    s.sc = word;
}

__device__ __forceinline__ void store_stage(const Stage& s, uint8_t* la, uint8_t* lb,
                                            uint32_t* lsa, uint32_t* lsb) {
    const int t = threadIdx.x;
    const int seg = t & 3;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = (t >> 2) + h * 64;
        *reinterpret_cast<u32x4_t*>(la + r * kLdsRow + seg * 16) = s.a[h];
        *reinterpret_cast<u32x4_t*>(lb + r * kLdsRow + seg * 16) = s.b[h];
    }
    if (t < 128) lsa[t] = s.sc;
    else lsb[t - 128] = s.sc;
}

// Round-to-nearest-even binary32 -> bf16 bits.
__device__ __forceinline__ uint32_t to_bf16(float f) {
    const uint32_t b = __float_as_uint(f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(kThreads) void k_gemm_mxfp4(GParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t s_a[2][BM * kLdsRow];
    __shared__ __attribute__((aligned(16))) uint8_t s_b[2][BN * kLdsRow];
    __shared__ uint32_t s_sa[2][BM];
    __shared__ uint32_t s_sb[2][BN];
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    // Tiles along N vary fastest, so consecutive workgroups share A's rows.
    const int64_t tiles_n = (p.N + BN - 1) / BN;
    const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * BM;
    const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * BN;
    const int64_t rows_a = p.M - m0 < BM ? p.M - m0 : BM;
    const int64_t rows_b = p.N - n0 < BN ? p.N - n0 : BN;
    Tiles w;
    w.a = make_rsrc(p.a_codes + m0 * (p.K / 2), rows_a * (p.K / 2));
    w.b = make_rsrc(p.b_codes + n0 * (p.K / 2), rows_b * (p.K / 2));
    w.sa = make_rsrc(p.a_scales + m0 * (p.K / 32), rows_a * (p.K / 32));
    w.sb = make_rsrc(p.b_scales + n0 * (p.K / 32), rows_b * (p.K / 32));

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const int64_t n_stages = (p.K + BK - 1) / BK;
    Stage st;
    load_stage(st, p, w, 0);
    store_stage(st, s_a[0], s_b[0], s_sa[0], s_sb[0]);
    const int fr = lane & 15, fk = lane >> 4;  // fragment row and K block of this lane
    for (int64_t s = 0; s < n_stages; ++s) {
        const int cur = (int)(s & 1);
        __syncthreads();  // stage s is in LDS; every wave is done with stage s - 1
        const bool more = s + 1 < n_stages;
        if (more) load_stage(st, p, w, (s + 1) * BK);
        v8i af[4], bf[4];
        int sa[4], sb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ra_row = wm * 64 + i * 16 + fr;
            const v4i v = *reinterpret_cast<const v4i*>(&s_a[cur][ra_row * kLdsRow + fk * 16]);
            af[i] = v8i{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
            sa[i] = (int)((s_sa[cur][ra_row] >> (8 * fk)) & 0xFFu);
            const int rb_row = wn * 64 + i * 16 + fr;
            const v4i w = *reinterpret_cast<const v4i*>(&s_b[cur][rb_row * kLdsRow + fk * 16]);
            bf[i] = v8i{w[0], w[1], w[2], w[3], 0, 0, 0, 0};
            sb[i] = (int)((s_sb[cur][rb_row] >> (8 * fk)) & 0xFFu);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af[i], bf[j], acc[i][j], kFmtE2M1, kFmtE2M1, 0, sa[i], 0, sb[j]);
        if (more) store_stage(st, s_a[cur ^ 1], s_b[cur ^ 1], s_sa[cur ^ 1], s_sb[cur ^ 1]);
    }

    // Lane l holds C[row0 + 4 (l / 16) + r][col0 + l % 16] of each 16 x 16 tile.
    const int eb = p.ct == 1 ? 4 : 2;
    const Rsrc rc = make_rsrc(static_cast<char*>(p.c) + m0 * p.N * eb, rows_a * p.N * eb);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + wn * 64 + j * 16 + fr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wm * 64 + i * 16 + 4 * fk + r;  // within the tile
                const bool in = row < rows_a && col < p.N;
                const int off = in ? (int)((row * p.N + col) * eb) : kDropped;
                if (p.ct == 1)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), rc, off, 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)to_bf16(acc[i][j][r]), rc,
                                                          off, 0, 0);
            }
        }
    }
}

}  // namespace

int launch_gemm(const GemmJob& j, char* msg, size_t msg_len) {
    if (j.M == 0 || j.N == 0) return 0;
    GParams p{j.a_codes, j.a_scales, j.b_codes, j.b_scales, j.M, j.N, j.K, j.c, j.ct};
    const int64_t tiles = ((j.M + BM - 1) / BM) * ((j.N + BN - 1) / BN);
    hipLaunchKernelGGL(k_gemm_mxfp4, dim3((unsigned)tiles), dim3(kThreads), 0,
                       static_cast<hipStream_t>(j.stream), p);
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess) return 0;
    snprintf(msg, msg_len, "gemm kernel launch: %s", hipGetErrorString(e));
    return (int)e;
}

}  // namespace fp4q
