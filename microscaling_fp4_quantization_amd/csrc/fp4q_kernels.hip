// fp4q_kernels.hip -- gfx950 kernels for block-wise microscaling FP4 quantization.
//
// Work layout.  A tensor of n = rows * cols elements is a flat run of n / b
// blocks (blocks never cross a row because cols % b == 0).  Each lane owns 8
// consecutive elements (one 16-byte load of bf16, two of fp32), so a block of b
// spans L = b / 8 lanes of one wavefront and a 64-lane wave covers a 512-element
// chunk with perfectly coalesced loads and 4-byte code stores.  Block maxima and
// error sums are reduced across the L lanes with DPP quad permutes and row
// mirrors; nothing goes through LDS on the hot path.  Waves take groups of
// chunks with every load of a group issued before any use (the split between
// waves and their numbering across the XCDs are chosen per kernel, see
// wave_range).  Memory is reached through
// range-checked buffer resources, so ragged ends need no branches.
//
// Arithmetic (the rules the pages leave open are stated in include/fp4q.h):
//   MXFP4: the E8M0 byte is the block maximum's binary32 exponent field minus 2
//   (clamped at 0); codes come from v_cvt_scalef32_pk_fp4_{bf16,f32}, which
//   divide by the scale's power of two exactly and round to nearest-even onto
//   E2M1 with saturation and a kept sign; dequantization (exact) from
//   v_cvt_scalef32_pk_f32_fp4.
//   UE4M3/UE5M3: s = m / D and the reciprocal r = 1 / d are correctly rounded
//   divisions once per block; the element quotient RN32(x / d) uses the
//   FMA-corrected reciprocal product of Markstein (IBM J. Res. Dev. 34(1), 1990):
//   q = x r, n = fma(q, d, -x), y = fma(-n, r, q), which returns the correctly
//   rounded quotient when r = RN(1/d) and no intermediate leaves the normal
//   range (the negated remainder keeps the sign of a zero quotient); blocks
//   whose d or x / d leave the safe range use a plain division.  y is then coded with the same cvt instruction at scale 1.
//   Errors: e = x - x_hat in binary32 (exact for MXFP4 and for unsaturated
//   UE4M3 blocks), squared and summed in binary64.  The sum of squares of x
//   (relative MSE, tensor term) is binary64 too, except for bf16 values
//   without rotation: their squares are exact in binary32 and the block's sum
//   is formed there, within (4 + log2 L) 2^-24 relatively (see sumsq_b32).  The max-element term is
//   computed from the block maximum m itself (every element attaining m has
//   the same error).  The non-max term is block SSE minus it when that
//   difference keeps at least 2^-12 of the SSE (then it is within b 2^-41 of
//   the separate sum, relatively); otherwise it is summed separately, element
//   by element, leaving out the lowest-index element attaining m (see
//   needs_separate_sum).
//   Tensor terms: per-workgroup binary64 partials, summed in a fixed order by a
//   one-workgroup finalize kernel (one workgroup per tensor for a batch), so
//   results are bit-reproducible.
//
// Launch forms.  k_quantize covers one tensor with the whole grid;
// k_quantize_amax is its MXFP4 form that also leaves per-workgroup maxima (the
// NVFP4 per-tensor scale of fp4_quantize_mx_nv without an amax pass);
// k_quantize_mx_batch / k_quantize_nv_batch cover up to 16 tensors in one
// launch, each tensor on its own run of workgroups.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "fp4q_launch.h"

namespace fp4q {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kLaneElems = 8;
constexpr int kChunk = kWave * kLaneElems;  // 512 elements per wave per chunk
#ifndef FP4Q_WAVES
#define FP4Q_WAVES 4
#endif
constexpr int kWaves = FP4Q_WAVES;
constexpr int kThreads = kWave * kWaves;
#ifndef FP4Q_STORE_NT
#define FP4Q_STORE_NT 0
#endif
#ifndef FP4Q_PREFETCH
#define FP4Q_PREFETCH 1
#endif
#ifndef FP4Q_LOAD_NT
#define FP4Q_LOAD_NT 1
#endif
#ifndef FP4Q_UNROLL
#define FP4Q_UNROLL 4
#endif
constexpr int kUnroll = FP4Q_UNROLL;        // chunks per wave iteration
#ifndef FP4Q_QUNROLL
#define FP4Q_QUNROLL 2
#endif
#ifndef FP4Q_AUNROLL
#define FP4Q_AUNROLL 4
#endif
constexpr int kQuantUnroll = FP4Q_QUNROLL;  // ... of the quantize kernel
constexpr int kAmaxUnroll = FP4Q_AUNROLL;   // ... of the amax pre-pass
// Quantize and amax grids: at least this many chunks per wave, and at most
// kGridRounds rounds of resident workgroups.
#ifndef FP4Q_MIN_CHUNKS_PER_WAVE
#define FP4Q_MIN_CHUNKS_PER_WAVE 4
#endif
#ifndef FP4Q_GRID_ROUNDS
#define FP4Q_GRID_ROUNDS 1
#endif
constexpr int kMinChunksPerWave = FP4Q_MIN_CHUNKS_PER_WAVE;
// Work split of the streaming kernels (see split_for): chunks per wave of
// short-lived workgroups (> 0), the balanced one-round split (0) or the
// one-round sweep (< 0).  Launches that leave per-workgroup partials (tensor
// stats) or reduce the amax pass in every workgroup (dynamic g) take the
// one-round grid: with short-lived workgroups those would be repeated by
// thousands of workgroups (measured: NVFP4 with stats 45 -> 54 us per 67.9 M
// elements).  UE-scale quantization, dequantization, rotation and block MSE
// without them take short-lived workgroups, which the dispatcher hands out in
// order as slots free up (interleaved medians on 67.9 M elements, two boxes:
// NVFP4 with per-block MSE 36.0-39.0 -> 34.8-35.4 us, fp32 dequantization
// 88.9 -> 80.1, rotation 97.4 -> 84.6, block MSE 40.3 -> 37.1); MXFP4
// quantization keeps the sweep (codes only: 31.2 against 33.2 us).
#ifndef FP4Q_QCPW
#define FP4Q_QCPW -1
#endif
#ifndef FP4Q_QCPW_LIGHT
#define FP4Q_QCPW_LIGHT 4
#endif
#ifndef FP4Q_ACPW
#define FP4Q_ACPW 8
#endif
// Smaller tensors give the amax pass fewer chunks per wave, so that it runs as
// one round of loads on more CUs (below this many chunks).
#ifndef FP4Q_ACPW_SMALL
#define FP4Q_ACPW_SMALL 4
#endif
#ifndef FP4Q_ACPW_SMALL_BELOW
#define FP4Q_ACPW_SMALL_BELOW 32768
#endif
#ifndef FP4Q_SCPW
#define FP4Q_SCPW 0
#endif
#ifndef FP4Q_SCPW_LIGHT
#define FP4Q_SCPW_LIGHT 4
#endif
constexpr int kQuantCpw = FP4Q_QCPW, kQuantCpwLight = FP4Q_QCPW_LIGHT, kAmaxCpw = FP4Q_ACPW;
constexpr int kAmaxCpwSmall = FP4Q_ACPW_SMALL;
constexpr int64_t kAmaxSmallBelow = FP4Q_ACPW_SMALL_BELOW;
constexpr int kStreamCpw = FP4Q_SCPW, kStreamCpwLight = FP4Q_SCPW_LIGHT;
// The amax pre-pass has no per-workgroup set-up, so it runs larger workgroups
// of short-lived waves: fewer per-workgroup maxima for the quantize kernel to
// reduce at the same wave count.
#ifndef FP4Q_AMAX_WAVES
#define FP4Q_AMAX_WAVES 16
#endif
constexpr int kAmaxWaves = FP4Q_AMAX_WAVES;

constexpr int kAmaxThreads = kWave * kAmaxWaves;
constexpr int kGridRounds = FP4Q_GRID_ROUNDS;

// The quantize and block-MSE kernels are held to 80 scalar registers.  At 96
// (the next allocation granule) fewer of their waves fit per SIMD on gfx950
// (measured on 70.8 M-element launches: mean occupancy 19.9 -> 14.0 waves per
// CU and 36 -> 45 us for MXFP4 with per-block MSE), while the occupancy query
// that sizes the one-round grids does not see that limit.  The few scalars
// over the cap go to VGPR lanes.
#define FP4Q_SGPR_CAP __attribute__((amdgpu_num_sgpr(80)))

constexpr int kFmtMx = 0;
constexpr int kFmtUe4m3 = 1;
constexpr int kFmtUe5m3 = 2;
constexpr int kMseRel = 1;

// DPP controls (GFX9 encoding).
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kRowMirror = 0x140;     // lane i <- lane 15-i within 16

constexpr uint32_t kRsqrt32Bits = 0x3E3504F3u;  // RN32(2^-2.5)

// ------------------------------------------------------------ lane helpers
// Every control used here reads a lane of the same row, so the row/bank masks
// and bound_ctrl never take effect; written as an update with old = 0 and
// bound_ctrl set, the move folds into the ALU instruction that uses it
// (v_max_u32_dpp, v_add_f32_dpp) instead of costing one of its own.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    uint64_t u = (uint64_t)__double_as_longlong(v);
    uint32_t lo = dpp_u32<CTRL>((uint32_t)u), hi = dpp_u32<CTRL>((uint32_t)(u >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Max over the L lanes of an aligned lane group; every lane gets the result.
template <int L>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
    if constexpr (L >= 2) v = max(v, dpp_u32<kQuadXor1>(v));
    if constexpr (L >= 4) v = max(v, dpp_u32<kQuadXor2>(v));
    if constexpr (L >= 8) v = max(v, dpp_u32<kRowHalfMirror>(v));
    if constexpr (L >= 16) v = max(v, dpp_u32<kRowMirror>(v));
    if constexpr (L >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16));
    return v;
}

template <int L>
__device__ __forceinline__ uint32_t group_min(uint32_t v) {
    if constexpr (L >= 2) v = min(v, dpp_u32<kQuadXor1>(v));
    if constexpr (L >= 4) v = min(v, dpp_u32<kQuadXor2>(v));
    if constexpr (L >= 8) v = min(v, dpp_u32<kRowHalfMirror>(v));
    if constexpr (L >= 16) v = min(v, dpp_u32<kRowMirror>(v));
    if constexpr (L >= 32) v = min(v, (uint32_t)__shfl_xor((int)v, 16));
    return v;
}

// Sum over the lane group.  Each step adds two equal-sized partial sums, so
// every lane ends with bit-identical totals.
template <int L>
__device__ __forceinline__ double group_sum(double v) {
    if constexpr (L >= 2) v = v + dpp_f64<kQuadXor1>(v);
    if constexpr (L >= 4) v = v + dpp_f64<kQuadXor2>(v);
    if constexpr (L >= 8) v = v + dpp_f64<kRowHalfMirror>(v);
    if constexpr (L >= 16) v = v + dpp_f64<kRowMirror>(v);
    if constexpr (L >= 32) v = v + __shfl_xor(v, 16);
    return v;
}

template <int L>
__device__ __forceinline__ float group_sum_f32(float v) {
    if constexpr (L >= 2) v = v + dpp_f32<kQuadXor1>(v);
    if constexpr (L >= 4) v = v + dpp_f32<kQuadXor2>(v);
    if constexpr (L >= 8) v = v + dpp_f32<kRowHalfMirror>(v);
    if constexpr (L >= 16) v = v + dpp_f32<kRowMirror>(v);
    if constexpr (L >= 32) v = v + __shfl_xor(v, 16);
    return v;
}

// A block's sum of squares (every lane of the block gets it), in binary64:
// exact squares, rounded only by the sum (relative error about b 2^-53).
template <int L>
__device__ __forceinline__ double sumsq_b64(const float (&v)[8]) {
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const double xv = (double)v[i];
        ss = fma(xv, xv, ss);
    }
    return group_sum<L>(ss);
}

// The same sum for values of 8 significant bits (bf16 inputs, no rotation)
// whose block maximum m passes sumsq_b32_ok, in binary32 at a third of the
// instructions.  Each square has at most 16 significant bits, so the products
// are exact; the lane's two interleaved chains of four (3 roundings each),
// their sum (1) and the log2 L cross-lane levels round every term at most
// 4 + log2 L times, so the result is within (4 + log2 L) 2^-24 of the exact
// sum, relatively (non-negative terms): at most 9 2^-24 = 5.4e-7 for b = 256.
// The window for m keeps m^2 and the block's sum normal and finite; smaller
// elements of the block whose squares fall below the normal range add an
// absolute error of at most 2^-150 each against a sum of at least 2^-100.
template <int L>
__device__ __forceinline__ double sumsq_b32(const float (&v)[8]) {
    float a = v[0] * v[0], b = v[1] * v[1];
    a = fmaf(v[2], v[2], a);
    b = fmaf(v[3], v[3], b);
    a = fmaf(v[4], v[4], a);
    b = fmaf(v[5], v[5], b);
    a = fmaf(v[6], v[6], a);
    b = fmaf(v[7], v[7], b);
    return (double)group_sum_f32<L>(a + b);
}

// Block maximum bits (binary32 of |x|) inside [2^-50, 2^60): the binary32 sum
// of squares applies (zero blocks and every other block take binary64).
__device__ __forceinline__ bool sumsq_b32_ok(uint32_t mbits) {
    constexpr uint32_t kLo = 77u << 23, kHi = 187u << 23;  // 2^-50, 2^60
    return mbits - kLo < kHi - kLo;
}

// A block's sum of squares as every kernel that forms one takes it (quantize,
// block MSE, scale search), so that their per-block results agree bit for bit:
// binary32 (sumsq_b32) for bf16 values without rotation (B32) whose block
// maximum, with binary32 bits mbits, passes sumsq_b32_ok; binary64 otherwise.
// The choice is the same on every lane of a block.
template <int L, bool B32>
__device__ __forceinline__ double block_sumsq(const float (&v)[8], uint32_t mbits) {
    if constexpr (B32) {
        if (sumsq_b32_ok(mbits)) return sumsq_b32<L>(v);
    }
    return sumsq_b64<L>(v);
}

__device__ __forceinline__ double wave_sum(double v) {
    for (int s = 32; s >= 1; s >>= 1) v = v + __shfl_xor(v, s);
    return v;
}

__device__ __forceinline__ long long wave_sum_i64(long long v) {
    for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s);
    return v;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    for (int s = 32; s >= 1; s >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, s));
    return v;
}

// Logical slice index for workgroup `bid` of `G`: workgroups are dispatched
// round-robin over the 8 XCDs, so XCD x receives bids x, x+8, ...; giving those
// consecutive slices keeps each XCD on one contiguous eighth of the tensor.
__device__ __forceinline__ int xcd_slice(int bid, int G) {
    const int q = G / 8, r = G % 8, x = bid % 8, k = bid / 8;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + k;
}

// ------------------------------------------------------------ input chunks
template <int XT>
struct Raw;
template <>
struct Raw<0> {  // 8 bf16
    uint4 w;
};
template <>
struct Raw<1> {  // 8 fp32
    uint4 a, b;
};

// ------------------------------------------------------------ buffer resources
// The hot kernels address memory through raw buffer resources (base, size in
// bytes) built per chunk group in scalar registers.  The hardware range check
// then does the bounds work: a load past the size returns zeros without
// touching memory and a store past it is dropped, so the ragged end of a
// tensor and the leader-only stores need no per-lane branches, and lane
// addresses are 32-bit offsets from a wave-uniform base.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;       // raw (stride 0) buffer, 32-bit data format
constexpr int kDropped = (int)0x80000000;    // an offset past every range: access dropped
constexpr int kNt = FP4Q_LOAD_NT ? 2 : 0;    // cache policy: nontemporal (read-once data)
// The NVFP4 pass of a batched combined call sweeps each tensor from its end
// to its start: the MXFP4 pass before it swept forward, so the part of the
// tensors still in the last-level cache is their end, which the NVFP4 pass
// then reads first, before its own output stores can evict it (one box, two
// interleaved rounds of the 48-layer step: NVFP4 launches 97.7 -> 92.7 us
// in the one-stream replay, the step 3736 -> 3743 GB/s).
#ifndef FP4Q_NV_BATCH_CPW
#define FP4Q_NV_BATCH_CPW -2
#endif
// Load policy of the combined calls' MXFP4 pass (see quantize_body): any
// policy without the nontemporal bit measured the same (SC0, SC1, both).
#ifndef FP4Q_MX_IN_POL
#define FP4Q_MX_IN_POL 0
#endif
constexpr int kStNt = FP4Q_STORE_NT ? 2 : 0;
// Store policy of the quantize outputs: UE-scale formats store with the SC1
// scope bit (interleaved medians on 67.9 M-element NVFP4 launches: 0.6-1.5 us
// faster in all three modes); MXFP4 keeps the default (0.5 us slower with it).
template <int FMT>
constexpr int quant_store_policy() { return FMT == kFmtMx ? kStNt : 16; }
// Store policy of the NVFP4 pass of a batched combined call: nontemporal.
// With SC1 its outputs stayed in the last-level cache and the next call's
// MXFP4 pass, which reads with the caching policy, ran slower (48-layer step,
// two interleaved rounds on one box: 3814 -> 4072 GB/s; in the one-stream
// replay MXFP4 launches 122.6 -> 106.1 us, NVFP4 94.1 -> 96.6 us).  SC1 with
// NT measured 1.4% below NT alone, SC0 with NT the same, and NT on the MXFP4
// pass's stores as well 0.6% below.
#ifndef FP4Q_BATCH_NV_STORE_POL
#define FP4Q_BATCH_NV_STORE_POL 2
#endif
constexpr int kBatchNvStore = FP4Q_BATCH_NV_STORE_POL;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

template <int POL = kNt>
__device__ __forceinline__ uint4 buf_load16(Rsrc r, int off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POL);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Work split shared by the streaming kernels.  The tensor is a run of C
// 512-element chunks; a wave takes n groups of up to kUnroll chunks, starting
// at chunks c0, c0 + step, ... (step may be negative), each clipped at c1:
//   cpw > 0: its own range [wid * cpw, (wid + 1) * cpw) (clipped to C), on a
//            grid of ceil(C / (4 cpw)) workgroups that may take several rounds;
//   cpw = 0: wave wid of W owns [wid * C / W, (wid + 1) * C / W), ranges within
//            one chunk of each other's length, for a one-round grid;
//   cpw < 0: groups wid, wid + W, wid + 2W, ... of the whole tensor on a
//            one-round grid, so that all waves sweep the tensor together and
//            the accesses in flight stay within a compact region; cpw = -2
//            sweeps from the end of the tensor to its start.
// With cpw != 0, waves are numbered in dispatch order (consecutive
// workgroups run on different XCDs; measured on 67.9 M elements against
// XCD-contiguous numbering: short-lived NVFP4 quantize 34.7 -> 33.0 us,
// rotation 84.6 -> 76.6 us, fp32 dequantization 80.5 -> 77.3 us; the sweeps
// 1-2.5 % faster); with cpw = 0 each XCD owns one contiguous eighth of the
// tensor.
struct WaveRange {
    int64_t c0, step, n, c1;
};

// The workgroups working on the tensor are wg_first .. wg_first + wg_count - 1
// of the grid (wg_count <= 0: the whole grid; a batched launch gives each
// tensor its own run of workgroups).
template <int WAVES = kWaves, int U = kUnroll>
__device__ __forceinline__ WaveRange wave_range(int64_t n_chunks, int64_t cpw, int wg_first = 0,
                                                int wg_count = 0) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int bid = (int)blockIdx.x - wg_first;
    const int G = wg_count > 0 ? wg_count : (int)gridDim.x;
    const int64_t W = (int64_t)G * WAVES;
    // Short-lived workgroups (cpw > 0) and the sweep (cpw < 0) keep the
    // dispatch order, so that the waves working at one time on all eight XCDs
    // cover one compact window of the tensor; the balanced split gives each
    // XCD a contiguous part.
    const int64_t slot = cpw != 0 ? (int64_t)bid : (int64_t)xcd_slice(bid, G);
    const int64_t wid = slot * WAVES + wave;
    if (cpw < 0) {
        const int64_t groups = (n_chunks + U - 1) / U;
        const int64_t n = wid < groups ? (groups - wid + W - 1) / W : 0;
        if (cpw == -2) return {(groups - 1 - wid) * U, -W * U, n, n_chunks};
        return {wid * U, W * U, n, n_chunks};
    }
    int64_t c0, c1;
    if (cpw > 0) {
        c0 = wid * cpw < n_chunks ? wid * cpw : n_chunks;
        c1 = c0 + cpw < n_chunks ? c0 + cpw : n_chunks;
    } else {
        c0 = wid * n_chunks / W;
        c1 = (wid + 1) * n_chunks / W;
    }
    return {c0, U, (c1 - c0 + U - 1) / U, c1};
}

// Loads the kUnroll chunks starting at chunk c; chunks at or past c1 (another
// wave's) and elements past n read as zeros.
// Input window of the U-chunk group starting at chunk c, clipped at chunk c1
// and at element n.
template <int XT, int U = kUnroll>
__device__ __forceinline__ Rsrc group_input(const void* x, int64_t n, int64_t c, int64_t c1) {
    constexpr int E = XT == 0 ? 2 : 4;
    const int64_t first = c * kChunk;
    int64_t avail = (c1 - c < U ? c1 - c : U) * kChunk;
    if (avail > n - first) avail = n - first;
    return make_rsrc(static_cast<const char*>(x) + first * E, avail * E);
}

template <int XT, int U = kUnroll>
__device__ __forceinline__ void load_group(Raw<XT> (&raw)[U], const void* x, int64_t n,
                                           int64_t c, int64_t c1, int lane) {
    constexpr int E = XT == 0 ? 2 : 4;
    const Rsrc r = group_input<XT, U>(x, n, c, c1);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if constexpr (XT == 0) {
            raw[u].w = buf_load16(r, u * kChunk * E + lane * 16);
        } else {
            raw[u].a = buf_load16(r, u * kChunk * E + lane * 32);
            raw[u].b = buf_load16(r, u * kChunk * E + lane * 32 + 16);
        }
    }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int XT>
__device__ __forceinline__ void unpack(const Raw<XT>& r, float (&v)[8]) {
    if constexpr (XT == 0) {
        v[0] = bf16_lo(r.w.x); v[1] = bf16_hi(r.w.x);
        v[2] = bf16_lo(r.w.y); v[3] = bf16_hi(r.w.y);
        v[4] = bf16_lo(r.w.z); v[5] = bf16_hi(r.w.z);
        v[6] = bf16_lo(r.w.w); v[7] = bf16_hi(r.w.w);
    } else {
        v[0] = __uint_as_float(r.a.x); v[1] = __uint_as_float(r.a.y);
        v[2] = __uint_as_float(r.a.z); v[3] = __uint_as_float(r.a.w);
        v[4] = __uint_as_float(r.b.x); v[5] = __uint_as_float(r.b.y);
        v[6] = __uint_as_float(r.b.z); v[7] = __uint_as_float(r.b.w);
    }
}

// ------------------------------------------------------------ rotation
// Normalised Sylvester Walsh-Hadamard transform of a block of ROT = 16 or 32
// values spread over ROT/8 lanes (gl = lane index within the block): stages
// h = 1, 2, 4 inside the lane, h = 8 and 16 across lanes, then the multiply by
// RN32(ROT^-1/2).  Across lanes the upper partner forms (partner - own) as
// fma(own, -1, partner), a single rounding of the same difference.
template <int ROT>
__device__ __forceinline__ void rotate8(float (&v)[8], int gl) {
#pragma unroll
    for (int h = 1; h < 8; h *= 2) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i & h) continue;
            const float a = v[i], b = v[i + h];
            v[i] = a + b;
            v[i + h] = a - b;
        }
    }
    const float s1 = (gl & 1) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = fmaf(v[i], s1, dpp_f32<kQuadXor1>(v[i]));
    if constexpr (ROT == 32) {
        const float s2 = (gl & 2) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = fmaf(v[i], s2, dpp_f32<kQuadXor2>(v[i]));
    }
    const float c = (ROT == 16) ? 0.25f : __uint_as_float(kRsqrt32Bits);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = v[i] * c;
}

// ------------------------------------------------------------ scale codes
// Round s >= 0 to the nearest UE4M3 (fmt 1) or UE5M3 (fmt 2) value, ties to
// the even code, saturating at the largest finite value.  Above the smallest
// normal value the binary32 significand is rounded to 3 bits in place (the
// rounded bits then read directly as the byte, after removing the exponent
// bias difference); below it the value is a multiple of the subnormal step.
__device__ __forceinline__ uint32_t ue5m3_encode(float s) {
    const uint32_t b = __float_as_uint(s);
    const uint32_t normal = ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - 896u;
    const uint32_t sub = (uint32_t)__builtin_rintf(s * 0x1p17f);
    const uint32_t byte = s < 0x1p-14f ? sub : normal;
    return min(byte, 0xF7u);
}

// UE4M3 uses the hardware OCP E4M3 conversion (round to nearest even, with
// subnormals); it gives the NaN code 0x7F from 464 up instead of saturating,
// so the byte is clamped to 0x7E (448).
__device__ __forceinline__ uint32_t ue_encode(float s, int fmt) {
    if (fmt == kFmtUe4m3)
        return min((uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s, 0.0f, 0, false) & 0xFFu, 0x7Eu);
    return ue5m3_encode(s);
}

__device__ __forceinline__ float ue_decode(uint32_t byte, int fmt) {
    const bool e4 = (fmt == kFmtUe4m3);
    if (byte < 8u) return (float)byte * (e4 ? 0x1p-9f : 0x1p-17f);
    return __uint_as_float((byte + (e4 ? 960u : 896u)) << 20);
}

// Correctly rounded x / d from r = RN(1/d) (Markstein's FMA correction),
// written with the negated remainder n = q d - x so that x = -0 gives -0.
// Exact whenever d is in [2^-96, 2^100] and |x / d| <= 4096 (and for d = 0
// with r = 0, where it yields a zero of x's sign).
__device__ __forceinline__ float div_rn(float x, float d, float r) {
    const float q = x * r;
    const float n = fmaf(q, d, -x);
    return fmaf(-n, r, q);
}

// Per-workgroup table of decode scales: for every scale byte c, d_c =
// RN32(s_hat_c * g), r_c = RN32(1 / d_c) (0 when d_c = 0) and lim_c, the
// largest block maximum for which the FMA-corrected quotients are exact:
// 4096 d_c when d_c is in [2^-96, 2^100], infinity when d_c = 0 (the quotients
// are then zeros of x's sign), and -1 (never) otherwise.  Only the saturating
// top code can exceed 4096 d_c; every other code has m / d_c below 9.
// The fourth entry is 1 when the block maximum is known to code to 6: c is a
// normal scale code and D = RN32(6 g) and d_c are normal binary32 numbers.
// Then s_hat_c is s rounded to 4 significant bits (relative error below 1/17,
// or s_hat_c < s when saturating) and D, d_c carry relative errors of at most
// 2^-24, so RN32(m / d_c) is about 6 s / s_hat_c > 5.6 and rounds to 6.
constexpr int kUeCodes = 256;  // covers UE4M3 (127 codes) and UE5M3 (248)

__device__ __forceinline__ void build_scale_table(float4* tab, float g, float D, int fmt) {
    const int n_codes = (fmt == kFmtUe4m3) ? 0x7F : 0xF8;
    for (int c = threadIdx.x; c < n_codes; c += kThreads) {
        const float d = ue_decode((uint32_t)c, fmt) * g;
        const float r = d > 0.0f ? 1.0f / d : 0.0f;
        float lim = -1.0f;
        if (d == 0.0f) lim = __builtin_inff();
        else if (d >= 0x1p-96f && d <= 0x1p100f) lim = d * 4096.0f;
        const bool six = c >= 8 && d >= 0x1p-126f && D >= 0x1p-126f;
        tab[c] = make_float4(d, r, lim, six ? 1.0f : 0.0f);
    }
    __syncthreads();
}

// Per-block UE scale state.
struct UeScale {
    uint32_t byte;
    float d, r;
    bool fast;  // the FMA-corrected quotient is exact for every element
    bool six;   // the block maximum codes to 6
};

// s = RN32(m / D): the corrected quotient when it is in its exact range (D in
// [2^-96, 2^100] and m / D <= 4096, which covers every unsaturated block),
// else a plain division.  s_fast_max is 4096 when D is in that range, else -1.
template <int FMT>
__device__ __forceinline__ UeScale ue_scale(float m, float D, float rD, float s_fast_max,
                                            const float4* tab) {
    UeScale st;
    float s = div_rn(m, D, rD);
    const bool slow = !(s <= s_fast_max);
    if (__builtin_amdgcn_ballot_w64(slow)) {  // wave-uniform: keeps the division off the fast path
        // The empty volatile asm pins the division inside the branch; without it
        // the compiler evaluates the full IEEE division on every block and selects.
        float mm = m;
        asm volatile("" : "+v"(mm));
        if (slow) s = mm / D;
    }
    st.byte = ue_encode(s, FMT);
    const float4 e = tab[st.byte];
    st.d = e.x;
    st.r = e.y;
    st.fast = m <= e.z;
    st.six = e.w != 0.0f;
    return st;
}

// Eight fp32 values -> one word of 8 codes (element 2k in byte k's low nibble).
__device__ __forceinline__ uint32_t code_word_f32(const float (&y)[8], float sc) {
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], sc, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], sc, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], sc, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], sc, 3);
    return w;
}

__device__ __forceinline__ uint32_t code_word_bf16(const uint4& w4, float sc) {
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2_t, w4.x), sc, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2_t, w4.y), sc, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2_t, w4.z), sc, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2_t, w4.w), sc, 3);
    return w;
}

// One word of 8 codes -> 8 values v * 2^exponent(sc).
__device__ __forceinline__ void decode_word(uint32_t w, float sc, float (&o)[8]) {
    float2_t t;
    t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 0); o[0] = t[0]; o[1] = t[1];
    t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 1); o[2] = t[0]; o[3] = t[1];
    t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 2); o[4] = t[0]; o[5] = t[1];
    t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 3); o[6] = t[0]; o[7] = t[1];
}

// Dequantized value of a single magnitude m under the block's scale.
__device__ __forceinline__ float requant_mx(float m, float sc) {
    const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, m, m, sc, 0);
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, sc, 0)[0];
}

__device__ __forceinline__ float requant_ue(float m, const UeScale& s) {
    const float y = s.fast ? div_rn(m, s.d, s.r) : m / s.d;
    const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y, y, 1.0f, 0);
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0)[0] * s.d;
}

// Relative block MSE, sse / ss rounded to binary32 (0 when ss = 0).  The
// reciprocal of ss comes from the hardware estimate and two Newton steps (each
// squares the relative error), so sse * r is within about 2^-51 of the exact
// quotient before the final rounding: the result is the correctly rounded
// quotient or, within 2^-51 of a rounding boundary, its neighbour (one binary32
// ulp).  ss is a sum of squares of binary32 values, so it lies in [2^-298,
// 2^264] when positive and neither it nor its reciprocal leaves the normal
// binary64 range.  This takes about half the instructions of the IEEE division.
__device__ __forceinline__ float rel_mse(double sse, double ss) {
    double r = __builtin_amdgcn_rcp(ss);
    r = fma(r, fma(-ss, r, 1.0), r);
    r = fma(r, fma(-ss, r, 1.0), r);
    return ss > 0.0 ? (float)(sse * r) : 0.0f;
}

// ------------------------------------------------------------ tensor terms
struct Acc {
    double nonmax = 0.0, max = 0.0, zero = 0.0, sumsq = 0.0;
    uint32_t nzero = 0;  // per lane: at most one per chunk the wave processes
    uint32_t fixup = 0;  // wave-uniform: a block's separate non-max sum was deferred
    uint32_t amax = 0;   // max |x| (binary32 bits) over the chunks quantized (k_quantize AMAX)
};

// How a chunk's blocks whose non-max term needs the separate sum
// (needs_separate_sum) are handled.  kSepInline sums them on the spot.
// kSepDefer adds 0 for them and raises acc.fixup; the wave then runs its range
// again in kSepFixup, which stores nothing and adds only those blocks'
// separate sums.  Deferring keeps that rarely run code out of the streaming
// loop (inline, its mere presence cost 5-9 us per 70.8 M-element launch).
constexpr int kSepInline = 0, kSepDefer = 1, kSepFixup = 2;

// Index within this lane (0..7) of the block's lowest-index element attaining
// the block maximum m, or 8 when another lane holds it.  Indices are kept
// lane-local so that no per-lane index constants stay live in registers.
template <int L>
__device__ __forceinline__ int lowest_max_in_lane(const float (&v)[8], float m, int gl) {
    uint32_t first = 8u;
#pragma unroll
    for (int i = 7; i >= 0; --i)
        if (fabsf(v[i]) == m) first = (uint32_t)i;
    const uint32_t key = group_min<L>(first == 8u ? 0xFFu : (uint32_t)gl * kLaneElems + first);
    return (key >> 3) == (uint32_t)gl ? (int)(key & 7u) : 8;
}

// The separate non-max sum from a lane's values v and dequantized values xh:
// the squared errors of every element but the lowest-index one attaining the
// block maximum m, summed in binary64 (each e^2 is exact there).  Every lane of
// the block gets the same total.
template <int L>
__device__ __forceinline__ double nonmax_sum(const float (&v)[8], const float (&xh)[8], float m,
                                             int gl) {
    const int skip = lowest_max_in_lane<L>(v, m, gl);
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const double e = (double)(v[i] - xh[i]);
        if (i != skip) s = fma(e, e, s);
    }
    return group_sum<L>(s);
}

// The non-max term of a block that is not zero-rounded is formed as nm =
// sse - M from its SSE and its max-element term M (one of the SSE's summands,
// so sse >= M).  sse is a binary64 sum of b exact squares, within b 2^-53 of
// the exact SSE, so when nm keeps at least 2^-12 of sse it is within b 2^-41
// (< 2^-33 for b <= 256) of the exact non-max sum, relatively.  Blocks whose
// maximum carries more of the error than that (rare: the other elements sit on
// or next to the grid) take the separate sum instead (nonmax_sum), in a
// wave-uniform branch or a fix-up pass (kSepDefer).  The decision is the same on every lane of a block.
__device__ __forceinline__ bool needs_separate_sum(bool zero, double sse, double nm) {
    return !zero && nm < sse * 0x1p-12;
}

// Adds one block's terms.  A zero-rounded block (m > 0, every x_hat = 0)
// contributes its SSE to the zero-rounding term; any other block contributes
// its max-element term and its non-max term.  Zero-rounded
// blocks are rare, so the selects run only in waves that hold one; the plain
// adds give the same sums for every other block.
__device__ __forceinline__ void add_block(Acc& acc, bool zero, double sse, double mterm,
                                          double nonmax, double ss) {
    if (__builtin_amdgcn_ballot_w64(zero)) {
        acc.zero += zero ? sse : 0.0;
        acc.nzero += zero ? 1u : 0u;
        acc.max += zero ? 0.0 : mterm;
        acc.nonmax += zero ? 0.0 : nonmax;
    } else {
        acc.max += mterm;
        acc.nonmax += nonmax;
    }
    acc.sumsq += ss;
}

// Where the tensor terms go: per-workgroup binary64 partials (structure of
// arrays, slot blockIdx.x of each term), summed in index order by k_finalize
// after the producing kernel.  (Summing them in the producing kernel's last
// workgroup needs a device-scope release per workgroup, which on this chip
// writes back every dirty L2 line of the XCD; with the output streams in
// flight that cost more than the separate kernel.)
struct StatsOut {
    double* partials;
    void* stats;               // fp4q_stats, or NULL (k_finalize then only forms g)
    long long n_blocks;
    const double* sumsq_part;  // sum x^2 of the amax pre-pass, or NULL
    int G_sumsq;
    // k_finalize of an MXFP4 pass that feeds an NVFP4 pass (fp4_quantize_mx_nv):
    // the per-tensor scale from the quantize kernel's per-workgroup maxima.
    const uint32_t* amax_part;
    int n_amax;
    float* g_out;              // NULL: no scale to form
};

// Fixed-order sum of G partials into the fp4q_stats struct, by one workgroup:
// thread i sums entries i, i + 256, ... of each term in index order, then a
// fixed butterfly within each wave and the waves in order.  Each batch loads 8
// entries of every term before adding any, so a batch costs one memory round
// trip.  When sumsq_part is given (the amax pre-pass computed sum x^2 in its
// G_sumsq workgroups), the sum x^2 term comes from it.
__device__ void sum_partials(const StatsOut& so, int G) {
    __shared__ double s_t[kWaves][4];
    __shared__ long long s_c[kWaves];
    constexpr int kBatch = 8;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const double* partials = so.partials;
    const double* ssq = so.sumsq_part ? so.sumsq_part : partials + 3 * (size_t)kMaxGroups;
    const int Gs = so.sumsq_part ? so.G_sumsq : G;
    const long long* cnt = reinterpret_cast<const long long*>(partials + 4 * (size_t)kMaxGroups);
    const int n_max = G > Gs ? G : Gs;
    double t[4] = {0.0, 0.0, 0.0, 0.0};
    long long c = 0;
    for (int b = threadIdx.x; b < n_max; b += kThreads * kBatch) {
        double v[4][kBatch];
        long long vc[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int i = b + q * kThreads;
            const int ig = i < G ? i : 0, is = i < Gs ? i : 0;
#pragma unroll
            for (int k = 0; k < 3; ++k) v[k][q] = partials[(size_t)k * kMaxGroups + ig];
            v[3][q] = ssq[is];
            vc[q] = cnt[ig];
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int i = b + q * kThreads;
            if (i < G) {
#pragma unroll
                for (int k = 0; k < 3; ++k) t[k] += v[k][q];
                c += vc[q];
            }
            if (i < Gs) t[3] += v[3][q];
        }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) t[k] = wave_sum(t[k]);
    c = wave_sum_i64(c);
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) s_t[wave][k] = t[k];
        s_c[wave] = c;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double* out = static_cast<double*>(so.stats);
        long long cz = 0;
        for (int k = 0; k < 4; ++k) {
            double s = 0.0;
            for (int w = 0; w < kWaves; ++w) s += s_t[w][k];
            out[k] = s;
        }
        for (int w = 0; w < kWaves; ++w) cz += s_c[w];
        reinterpret_cast<long long*>(out)[4] = so.n_blocks;
        reinterpret_cast<long long*>(out)[5] = cz;
    }
}

// Each workgroup writes its partial terms to slot blockIdx.x; the kernel
// boundary makes them visible to k_finalize on every XCD.
__device__ void write_partial(const Acc& a, const StatsOut& so) {
    __shared__ double s_acc[kWaves][4];
    __shared__ long long s_cnt[kWaves];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const double t0 = wave_sum(a.nonmax), t1 = wave_sum(a.max), t2 = wave_sum(a.zero),
                 t3 = wave_sum(a.sumsq);
    const long long tc = wave_sum_i64((long long)a.nzero);
    if (lane == 0) {
        s_acc[wave][0] = t0; s_acc[wave][1] = t1; s_acc[wave][2] = t2; s_acc[wave][3] = t3;
        s_cnt[wave] = tc;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int k = 0; k < 4; ++k) {
            double s = 0.0;
            for (int w = 0; w < kWaves; ++w) s += s_acc[w][k];
            so.partials[(size_t)k * kMaxGroups + blockIdx.x] = s;
        }
        long long c = 0;
        for (int w = 0; w < kWaves; ++w) c += s_cnt[w];
        reinterpret_cast<long long*>(so.partials + 4 * (size_t)kMaxGroups)[blockIdx.x] = c;
    }
}

// ------------------------------------------------------------ quantize
struct QParams {
    const void* x;
    int64_t n, n_chunks, n_blocks;
    int64_t cpw;  // chunks per wave, 0 = balanced one-round split
    uint8_t* codes;
    uint8_t* scales;
    float* block_mse;
    int mse_kind;
    int fmt;            // UE kernels: 1 UE4M3, 2 UE5M3
    int radius;         // scale search: neighbours of the max-based code tried
    int max_byte;       // scale search: largest valid scale code
    const float* g_in;  // per-tensor scale (device), NULL for g = 1
    // Dynamic mode: per-workgroup |x| maxima of the amax pass; every workgroup
    // reduces them to g, and workgroup 0 also writes g to g_out.
    const uint32_t* amax_part;
    int n_amax;
    float* g_out;
    uint32_t* amax_out;  // k_quantize AMAX: per-workgroup max |x| bits (slot blockIdx.x)
    // The tensor's workgroups within the grid (see wave_range); 0, 0 = all.
    int wg_first, wg_count;
    StatsOut so;
};

// Per-kernel UE scale context: g, D = RN32(6 g), rD = RN32(1 / D), whether the
// corrected quotient m / D is usable, and the workgroup's decode-scale table.
struct UeCtx {
    float g, D, rD;
    float s_fast_max;  // 4096 when D is in [2^-96, 2^100], else -1
    const float4* tab;
};

// Output windows of one chunk group (wave-uniform): codes, scale bytes and
// per-block MSE of the group's valid blocks.
struct QOut {
    Rsrc codes, scales, mse;
};

// The quantize loop's chunk arithmetic in 32 bits.  Chunk indices fit 31 bits
// (the library rejects tensors of more chunks), and the scalar unit has no
// ordered 64-bit comparison: with 64-bit indices every clip of a group window
// became VALU compares and moves.  Only a group that reaches the tensor's last
// chunk (index n_chunks - 1, holding `tail` elements) is short of whole
// chunks; c < c1 <= n_chunks.
struct Chunks32 {
    int n_chunks, tail;
};

__device__ __forceinline__ Chunks32 chunks32(int64_t n, int64_t n_chunks) {
    return {(int)n_chunks, (int)(n - (n_chunks - 1) * kChunk)};
}

template <int U>
__device__ __forceinline__ int group_elems(int c, int c1, const Chunks32& k) {
    const int cl = c1 - c < U ? c1 - c : U;
    return cl * kChunk - (c + cl == k.n_chunks ? kChunk - k.tail : 0);
}

template <int B, int U>
__device__ __forceinline__ QOut group_outputs32(const QParams& p, int c, int c1, const Chunks32& k) {
    const int64_t first = (int64_t)c * kChunk;
    const int avail = group_elems<U>(c, c1, k);
    QOut o;
    o.codes = make_rsrc(p.codes + first / 2, avail / 2);
    o.scales = make_rsrc(p.scales + first / B, avail / B);
    o.mse = make_rsrc(p.block_mse + first / B, p.block_mse ? avail / B * 4 : 0);
    return o;
}

template <int XT, int U>
__device__ __forceinline__ Rsrc group_input32(const void* x, int c, int c1, const Chunks32& k) {
    constexpr int E = XT == 0 ? 2 : 4;
    return make_rsrc(static_cast<const char*>(x) + (int64_t)c * kChunk * E,
                     group_elems<U>(c, c1, k) * E);
}

template <int XT, int U, int POL = kNt>
__device__ __forceinline__ void load_group32(Raw<XT> (&raw)[U], const void* x, int c, int c1,
                                             const Chunks32& k, int lane) {
    constexpr int E = XT == 0 ? 2 : 4;
    const Rsrc r = group_input32<XT, U>(x, c, c1, k);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if constexpr (XT == 0) {
            raw[u].w = buf_load16<POL>(r, u * kChunk * E + lane * 16);
        } else {
            raw[u].a = buf_load16<POL>(r, u * kChunk * E + lane * 32);
            raw[u].b = buf_load16<POL>(r, u * kChunk * E + lane * 32 + 16);
        }
    }
}

// One lane's raw values of the chunk that starts xoff bytes into window r.
template <int XT>
__device__ __forceinline__ Raw<XT> load_chunk(Rsrc r, int xoff, int lane) {
    Raw<XT> raw;
    if constexpr (XT == 0) {
        raw.w = buf_load16(r, xoff + lane * 16);
    } else {
        raw.a = buf_load16(r, xoff + lane * 32);
        raw.b = buf_load16(r, xoff + lane * 32 + 16);
    }
    return raw;
}

// The separate non-max sum of a chunk's blocks (see needs_separate_sum) for
// kSepInline, with the values read again from memory and their codes and
// dequantized values formed again, two elements at a time, as quantize_chunk
// forms them under the block's scale: its power of two (MXFP4) or its decode
// scale d (UE formats; the IEEE quotient x / d is the value the corrected
// quotient gives where that is used).  Only waves holding a block that needs
// it run this, and it keeps little live, since the kernels that sum inline
// hold a whole prefetched row group in registers.
template <int XT, int FMT, int B, int ROT>
__device__ __forceinline__ double nonmax_reread(Rsrc xin, int xoff, int lane, int gl, float m,
                                                float scale) {
    constexpr int L = B / kLaneElems;
    const Raw<XT> raw = load_chunk<XT>(xin, xoff, lane);
    float v[8];
    unpack<XT>(raw, v);
    if constexpr (ROT != 0) rotate8<ROT>(v, gl);
    const int skip = lowest_max_in_lane<L>(v, m, gl);
    const float sc = FMT == kFmtMx ? scale : 1.0f;
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
        // One pair at a time: the barrier keeps the scheduler from forming
        // all pairs at once (which would raise the kernel's register count).
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ROT == 0) {
            float w[8];
            unpack<XT>(raw, w);
            v[j] = w[j];
            v[j + 1] = w[j + 1];
        }
        uint32_t c;
        if constexpr (FMT == kFmtMx) {
            c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[j], v[j + 1], sc, 0);
        } else {
            const float y0 = v[j] / scale, y1 = v[j + 1] / scale;
            c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y0, y1, 1.0f, 0);
        }
        const float2_t h = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, sc, 0);
        float x0 = h[0], x1 = h[1];
        if constexpr (FMT != kFmtMx) {
            x0 = x0 * scale;
            x1 = x1 * scale;
        }
        const double e0 = (double)(v[j] - x0), e1 = (double)(v[j + 1] - x1);
        if (skip != j) s = fma(e0, e0, s);
        if (skip != j + 1) s = fma(e1, e1, s);
    }
    __builtin_amdgcn_sched_barrier(0);
    return group_sum<L>(s);
}

// What a block's MSE and tensor terms need from its chunk (PAIR mode of
// quantize_chunk): the block's SSE and sum of squares, its maximum |x| and that
// maximum's dequantized value.  An absent chunk is all zeros, which stores
// nothing (its offsets fall outside the group's output window) and adds 0.
struct BlockRes {
    double sse = 0.0, ss = 0.0;
    float m = 0.0f, xh_m = 0.0f;
};

// One 512-element chunk: lane `lane` holds elements 8 lane .. 8 lane + 7 of it
// and block lane / L of it (gl = lane % L).  Every lane of a block ends with the
// block's results; the block's first lane stores its scale and MSE, and every
// lane adds the block's terms to acc (the caller keeps one lane's copy per
// block: gl = 0, or gl = 0 and 1 in PAIR mode).
// The chunk's input starts xoff bytes into the window xin (read again only for
// the separate non-max sum in kSepInline).  SEP: see kSepInline.
// PAIR (blocks of L >= 2 lanes, two-chunk groups): the chunk stores its codes
// and scale bytes and hands its blocks' sums to `res`, and finish_pair then
// forms the MSE and tensor terms of both chunks at once; in kSepFixup only
// lane gl = u adds (the lane finish_pair gives chunk u's block).
template <int XT, int FMT, int B, int ROT, bool ERR, bool SUMSQ, int SEP = kSepInline,
          bool PAIR = false, int ST = quant_store_policy<FMT>()>
__device__ __forceinline__ void quantize_chunk(const Raw<XT>& raw, int u, const QOut& o,
                                               const QParams& p, const UeCtx& ue, int lane,
                                               int gl, Acc& acc, Rsrc xin, int xoff,
                                               BlockRes* res = nullptr) {
    constexpr int L = B / kLaneElems;
    constexpr int kBlocks = kChunk / B;
    constexpr int kSt = ST;
    constexpr bool kPackedBf16 = (XT == 0) && (ROT == 0);
    float v[8];
    uint32_t lane_max;
    if constexpr (kPackedBf16) {
        // |x| of bf16 orders like its integer bits: max with packed u16 ops
        const u16x2_t a0 = __builtin_bit_cast(u16x2_t, raw.w.x & 0x7FFF7FFFu);
        const u16x2_t a1 = __builtin_bit_cast(u16x2_t, raw.w.y & 0x7FFF7FFFu);
        const u16x2_t a2 = __builtin_bit_cast(u16x2_t, raw.w.z & 0x7FFF7FFFu);
        const u16x2_t a3 = __builtin_bit_cast(u16x2_t, raw.w.w & 0x7FFF7FFFu);
        const u16x2_t mm = __builtin_elementwise_max(__builtin_elementwise_max(a0, a1),
                                                     __builtin_elementwise_max(a2, a3));
        lane_max = (uint32_t)max(mm[0], mm[1]) << 16;
        if constexpr (ERR || FMT != kFmtMx) unpack<XT>(raw, v);
    } else {
        unpack<XT>(raw, v);
        if constexpr (ROT != 0) rotate8<ROT>(v, gl);
        float mf = fmaxf(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))),
                         fmaxf(fmaxf(fabsf(v[4]), fabsf(v[5])), fmaxf(fabsf(v[6]), fabsf(v[7]))));
        lane_max = __float_as_uint(mf);
    }
    const uint32_t mbits = group_max<L>(lane_max);
    const float m = __uint_as_float(mbits);
    if constexpr (SEP != kSepFixup) acc.amax = max(acc.amax, mbits);  // read only by k_quantize AMAX

    uint32_t cw, sbyte;
    float xh[8];
    float xh_m = 0.0f;
    if constexpr (FMT == kFmtMx) {
        // The scale's bits: the exponent field of m, less 2, clamped at 0.
        const uint32_t sc_bits = __builtin_elementwise_sub_sat(mbits & 0x7F800000u, 2u << 23);
        sbyte = sc_bits >> 23;
        const float sc = __uint_as_float(sc_bits);
        if constexpr (kPackedBf16) cw = code_word_bf16(raw.w, sc);
        else cw = code_word_f32(v, sc);
        if constexpr (ERR) {
            decode_word(cw, sc, xh);
            if (p.so.stats) xh_m = requant_mx(m, sc);
        }
    } else {
        const UeScale s = ue_scale<FMT>(m, ue.D, ue.rD, ue.s_fast_max, ue.tab);
        sbyte = s.byte;
        float y[8];
        if (s.fast) {
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = div_rn(v[i], s.d, s.r);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = v[i] / s.d;
        }
        cw = code_word_f32(y, 1.0f);
        if constexpr (ERR) {
            decode_word(cw, 1.0f, xh);
#pragma unroll
            for (int i = 0; i < 8; ++i) xh[i] = xh[i] * s.d;
            if (p.so.stats) {
                xh_m = 6.0f * s.d;  // the decoded code 6, as for the elements
                if (__builtin_amdgcn_ballot_w64(!s.six)) {
                    if (!s.six) xh_m = requant_ue(m, s);
                }
            }
        }
    }
    const int blk = u * kBlocks + lane / L;  // block index within the group
    if constexpr (SEP != kSepFixup) {
        __builtin_amdgcn_raw_buffer_store_b32(cw, o.codes, (u * kChunk + lane * kLaneElems) / 2, 0,
                                              kSt);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sbyte, o.scales, gl == 0 ? blk : kDropped, 0,
                                             kSt);
    }
    if constexpr (ERR) {
        double sse = 0.0, ss = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double e = (double)(v[i] - xh[i]);
            sse = fma(e, e, sse);
        }
        sse = group_sum<L>(sse);
        if constexpr (SUMSQ) ss = block_sumsq<L, kPackedBf16>(v, mbits);
        if constexpr (PAIR && SEP != kSepFixup) {
            *res = BlockRes{sse, ss, m, xh_m};
            return;
        }
        if (SEP != kSepFixup && p.block_mse) {
            float mse;
            // Relative MSE always comes with the sum of squares (SUMSQ).
            if (SUMSQ && p.mse_kind == kMseRel) mse = rel_mse(sse, ss);
            else mse = (float)(sse * (1.0 / B));
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(mse), o.mse,
                                                  gl == 0 ? blk * 4 : kDropped, 0, kSt);
        }
        // Zero-filled lanes past the end form all-zero blocks, which add 0 to
        // every term and are not zero-rounded (m = 0).  Without tensor stats
        // the terms are not formed at all (a wave-uniform branch).
        if (p.so.stats) {
            const double em = (double)(m - xh_m);
            const double mterm = em * em;
            const bool zero = (m > 0.0f) && (xh_m == 0.0f);
            double nm = sse - mterm;
            const bool sep = needs_separate_sum(zero, sse, nm);
            if constexpr (SEP == kSepInline) {
                if (__builtin_amdgcn_ballot_w64(sep)) {
                    const float scale = FMT == kFmtMx ? __uint_as_float(sbyte << 23)
                                                      : ue.tab[sbyte].x;
                    const double s2 = nonmax_reread<XT, FMT, B, ROT>(xin, xoff, lane, gl, m, scale);
                    if (sep) nm = s2;
                }
            } else if constexpr (SEP == kSepDefer) {
                if (sep) nm = 0.0;
                if (__builtin_amdgcn_ballot_w64(sep)) acc.fixup = 1u;
            } else {
                if (__builtin_amdgcn_ballot_w64(sep)) {
                    const double s2 = nonmax_sum<L>(v, xh, m, gl);
                    if (sep && (!PAIR || gl == u)) acc.nonmax += s2;
                }
                return;
            }
            add_block(acc, zero, sse, mterm, nm, ss);
        }
    }
}

// The block MSE and tensor terms of two chunks' blocks (PAIR mode), one block
// per lane: lane gl = 0 of each block position takes the first chunk's block
// and lane gl = 1 the second's.  The lanes gl >= 2 of wider blocks compute
// copies whose stores are dropped and whose terms the caller discards.  This
// runs the per-block arithmetic once per two chunks instead of once per chunk
// on every lane of every block.  Non-max sums that need the separate sum are
// deferred (kSepDefer).
template <int FMT, int B, bool SUMSQ, int ST = quant_store_policy<FMT>()>
__device__ __forceinline__ void finish_pair(const BlockRes (&r)[2], const QOut& o, const QParams& p,
                                            int lane, int gl, Acc& acc) {
    constexpr int L = B / kLaneElems;
    constexpr int kBlocks = kChunk / B;
    constexpr int kSt = ST;
    static_assert(L >= 2, "one block per lane needs no pairing");
    const bool second = (gl & 1) != 0;
    const double sse = second ? r[1].sse : r[0].sse;
    const float m = second ? r[1].m : r[0].m;
    const float xh_m = second ? r[1].xh_m : r[0].xh_m;
    double ss = 0.0;
    if constexpr (SUMSQ) ss = second ? r[1].ss : r[0].ss;
    if (p.block_mse) {
        float mse;
        if (SUMSQ && p.mse_kind == kMseRel) mse = rel_mse(sse, ss);
        else mse = (float)(sse * (1.0 / B));
        const int blk = (second ? kBlocks : 0) + lane / L;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(mse), o.mse, gl < 2 ? blk * 4 : kDropped,
                                              0, kSt);
    }
    if (p.so.stats) {
        const double em = (double)(m - xh_m);
        const double mterm = em * em;
        const bool zero = (m > 0.0f) && (xh_m == 0.0f);
        double nm = sse - mterm;
        const bool sep = needs_separate_sum(zero, sse, nm);
        if (sep) nm = 0.0;
        if (__builtin_amdgcn_ballot_w64(sep)) acc.fixup = 1u;
        add_block(acc, zero, sse, mterm, nm, ss);
    }
}

// Scale search on one chunk (SEP: kSepDefer or kSepFixup, see kSepInline).
// Candidates are the max-based scale code c0 (the
// code quantize_chunk takes) and its neighbours c0 + j, 0 < |j| <= radius,
// inside [0, max_byte]; consecutive codes are consecutive scale values in all
// three formats.  Each is scored by the block's SSE in binary64, with every
// element coded and dequantized as quantize_chunk does under that code and
// its error formed in binary64 (x - x_hat of two binary32 values is then
// exact, so the scores match a sequential sum to rounding far below the
// margin).  Candidates are visited as j = 0, -1, +1, -2, +2, ... and one
// replaces the best so far only when its SSE is below best - best * 2^-40, so
// near-ties keep the code closest to c0.  Outputs are quantize_chunk's, for
// the chosen code.
template <int XT, int FMT, int B, int ROT, bool SUMSQ, int SEP>
__device__ __forceinline__ void search_chunk(const Raw<XT>& raw, int u, const QOut& o,
                                             const QParams& p, const UeCtx& ue, int lane,
                                             int gl, Acc& acc) {
    constexpr int L = B / kLaneElems;
    constexpr int kBlocks = kChunk / B;
    constexpr int kSt = quant_store_policy<FMT>();
    float v[8];
    unpack<XT>(raw, v);
    if constexpr (ROT != 0) rotate8<ROT>(v, gl);
    const float mf = fmaxf(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))),
                           fmaxf(fmaxf(fabsf(v[4]), fabsf(v[5])), fmaxf(fabsf(v[6]), fabsf(v[7]))));
    const uint32_t mbits = group_max<L>(__float_as_uint(mf));
    const float m = __uint_as_float(mbits);
    int c0;
    if constexpr (FMT == kFmtMx) {
        const uint32_t F = mbits >> 23;
        c0 = F > 2u ? (int)F - 2 : 0;
    } else {
        c0 = (int)ue_scale<FMT>(m, ue.D, ue.rD, ue.s_fast_max, ue.tab).byte;
    }
    double best = 0.0;
    int best_byte = c0;
    uint32_t best_cw = 0;
    float best_xm = 0.0f;
    for (int t = 0; t <= 2 * p.radius; ++t) {  // the same trip count on every lane
        const int j = t == 0 ? 0 : ((t & 1) ? -((t + 1) >> 1) : (t >> 1));
        const bool valid = c0 + j >= 0 && c0 + j <= p.max_byte;
        const int cb = valid ? c0 + j : c0;  // an in-range code; its result is not taken
        uint32_t cw;
        float xh[8], xm;
        if constexpr (FMT == kFmtMx) {
            const float sc = __uint_as_float((uint32_t)cb << 23);
            cw = code_word_f32(v, sc);
            decode_word(cw, sc, xh);
            xm = p.so.stats ? requant_mx(m, sc) : 0.0f;
        } else {
            const float4 e = ue.tab[cb];
            UeScale s;
            s.byte = (uint32_t)cb;
            s.d = e.x;
            s.r = e.y;
            s.fast = m <= e.z;
            s.six = e.w != 0.0f;
            float y[8];
            if (s.fast) {
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] = div_rn(v[i], s.d, s.r);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] = v[i] / s.d;
            }
            cw = code_word_f32(y, 1.0f);
            decode_word(cw, 1.0f, xh);
#pragma unroll
            for (int i = 0; i < 8; ++i) xh[i] = xh[i] * s.d;
            xm = p.so.stats ? requant_ue(m, s) : 0.0f;
        }
        double sse = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double e = (double)v[i] - (double)xh[i];
            sse = fma(e, e, sse);
        }
        sse = group_sum<L>(sse);
        if (valid && (t == 0 || sse < best - best * 0x1p-40)) {
            best = sse;
            best_byte = cb;
            best_cw = cw;
            best_xm = xm;
        }
    }
    double ss = 0.0;
    if constexpr (SUMSQ) ss = block_sumsq<L, XT == 0 && ROT == 0>(v, __float_as_uint(m));
    const int blk = u * kBlocks + lane / L;
    if constexpr (SEP != kSepFixup) {
        __builtin_amdgcn_raw_buffer_store_b32(best_cw, o.codes, (u * kChunk + lane * kLaneElems) / 2,
                                              0, kSt);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)best_byte, o.scales, gl == 0 ? blk : kDropped,
                                             0, kSt);
    }
    if (SEP != kSepFixup && p.block_mse) {
        float mse;
        if (SUMSQ && p.mse_kind == kMseRel) mse = rel_mse(best, ss);
        else mse = (float)(best * (1.0 / B));
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(mse), o.mse,
                                              gl == 0 ? blk * 4 : kDropped, 0, kSt);
    }
    if (p.so.stats) {
        const double em = (double)(m - best_xm);
        const double mterm = em * em;
        const bool zero = (m > 0.0f) && (best_xm == 0.0f);
        double nm = best - mterm;
        const bool sep = needs_separate_sum(zero, best, nm);
        if constexpr (SEP == kSepDefer) {
            if (sep) nm = 0.0;
            if (__builtin_amdgcn_ballot_w64(sep)) acc.fixup = 1u;
        } else if constexpr (SEP == kSepFixup) {
            if (__builtin_amdgcn_ballot_w64(sep)) {
                float xh[8];  // the chosen code's dequantized values
                if constexpr (FMT == kFmtMx) {
                    decode_word(best_cw, __uint_as_float((uint32_t)best_byte << 23), xh);
                } else {
                    decode_word(best_cw, 1.0f, xh);
                    const float d = ue.tab[best_byte].x;
#pragma unroll
                    for (int i = 0; i < 8; ++i) xh[i] = xh[i] * d;
                }
                const double s2 = nonmax_sum<L>(v, xh, m, gl);
                if (sep) acc.nonmax += s2;
            }
            return;
        }
        add_block(acc, zero, best, mterm, nm, ss);
    }
}

// g = RN32(amax / 2688) (1 when that is not positive) from the amax pass's
// per-workgroup maxima; every workgroup reduces the same values in the same
// way, so all agree bit for bit.
__device__ float dynamic_g(const uint32_t* part, int n_part) {
    __shared__ uint32_t s_m[kWaves];
    uint32_t m = 0;
    for (int i = threadIdx.x; i < n_part; i += kThreads) m = max(m, part[i]);
    m = wave_max(m);
    if (threadIdx.x % kWave == 0) s_m[threadIdx.x / kWave] = m;
    __syncthreads();
    uint32_t mm = s_m[0];
    for (int w = 1; w < kWaves; ++w) mm = max(mm, s_m[w]);
    const float g = __uint_as_float(mm) / 2688.0f;
    return g > 0.0f ? g : 1.0f;
}

// Sums a stats kernel's G partials (when so.stats is set) and, for an MXFP4
// pass that feeds an NVFP4 pass, forms the per-tensor scale from its maxima.
__global__ __launch_bounds__(kThreads) void k_finalize(StatsOut so, int G) {
    if (so.g_out) {
        const float g = dynamic_g(so.amax_part, so.n_amax);
        if (threadIdx.x == 0) *so.g_out = g;
    }
    if (so.stats) sum_partials(so, G);
}

#ifndef FP4Q_QUANT_WPE
#define FP4Q_QUANT_WPE 0
#endif
// The quantize kernel's body.  AMAX: also write the workgroup's max |x|
// (binary32 bits) to p.amax_out.
template <int XT, int FMT, int B, int ROT, bool ERR, bool SUMSQ, bool SEARCH, bool AMAX,
          int ST = quant_store_policy<FMT>()>
__device__ __forceinline__ void quantize_body(const QParams& p) {
    constexpr int L = B / kLaneElems;
    const int lane = threadIdx.x % kWave;
    const int gl = lane & (L - 1);
    const WaveRange wr = wave_range<kWaves, kQuantUnroll>(p.n_chunks, p.cpw, p.wg_first, p.wg_count);
    const Chunks32 ck = chunks32(p.n, p.n_chunks);
    const int c0 = (int)wr.c0, cstep = (int)wr.step, n_groups = (int)wr.n, c1 = (int)wr.c1;
    // The first group's loads go out before the per-workgroup set-up below, so
    // that set-up overlaps their latency.
    Raw<XT> cur[kQuantUnroll];
    // The MXFP4 pass of a combined call (AMAX) reads its input with the
    // default cache policy instead of the streaming one, so that the NVFP4
    // pass that reads the same tensors next finds part of them in the
    // last-level cache.  48-layer step, two interleaved rounds on one box:
    // 3662 -> 3733 GB/s; in the one-stream replay the NVFP4 launches went
    // 117 -> 97 us and the MXFP4 ones 110.5 -> 125 us.  (Both passes on the
    // default policy: 3719 GB/s, NVFP4 116 us.)
    constexpr int kInPol = AMAX ? FP4Q_MX_IN_POL : kNt;
    if (n_groups > 0) load_group32<XT, kQuantUnroll, kInPol>(cur, p.x, c0, c1, ck, lane);
    UeCtx ue{1.0f, 6.0f, 0.0f, 4096.0f, nullptr};
    if constexpr (FMT != kFmtMx) {
        __shared__ float4 s_tab[kUeCodes];
        float g = 1.0f;
        if (p.amax_part) {
            g = dynamic_g(p.amax_part, p.n_amax);
            if ((int)blockIdx.x == p.wg_first && threadIdx.x == 0) *p.g_out = g;
        } else if (p.g_in) {
            g = *p.g_in;
        }
        ue.g = g;
        ue.D = 6.0f * g;
        ue.rD = 1.0f / ue.D;
        ue.s_fast_max = (ue.D >= 0x1p-96f && ue.D <= 0x1p100f) ? 4096.0f : -1.0f;
        build_scale_table(s_tab, g, ue.D, FMT);
        ue.tab = s_tab;
    }
    Acc acc;
    constexpr int E = XT == 0 ? 2 : 4;
    // Blocks of two or more lanes finish a group's two chunks together.
    constexpr bool kPair = ERR && !SEARCH && L >= 2 && kQuantUnroll == 2;
    for (int i = 0, c = c0; i < n_groups; ++i, c += cstep) {
        const QOut o = group_outputs32<B, kQuantUnroll>(p, c, c1, ck);
        const Rsrc xin = group_input32<XT, kQuantUnroll>(p.x, c, c1, ck);
        const int left = c1 - c;  // wave-uniform
        Raw<XT> nxt[kQuantUnroll];
        if (i + 1 < n_groups)
            load_group32<XT, kQuantUnroll, kInPol>(nxt, p.x, c + cstep, c1, ck, lane);
        if constexpr (kPair) {
            BlockRes r[2];
            quantize_chunk<XT, FMT, B, ROT, ERR, SUMSQ, kSepDefer, true, ST>(
                cur[0], 0, o, p, ue, lane, gl, acc, xin, 0, &r[0]);
            if (left > 1)
                quantize_chunk<XT, FMT, B, ROT, ERR, SUMSQ, kSepDefer, true, ST>(
                    cur[1], 1, o, p, ue, lane, gl, acc, xin, kChunk * E, &r[1]);
            if (p.block_mse || p.so.stats) finish_pair<FMT, B, SUMSQ, ST>(r, o, p, lane, gl, acc);
        } else {
#pragma unroll
            for (int u = 0; u < kQuantUnroll; ++u)
                if (u < left) {
                    if constexpr (SEARCH)
                        search_chunk<XT, FMT, B, ROT, SUMSQ, kSepDefer>(cur[u], u, o, p, ue, lane, gl,
                                                                        acc);
                    else
                        quantize_chunk<XT, FMT, B, ROT, ERR, SUMSQ, kSepDefer, false, ST>(
                            cur[u], u, o, p, ue, lane, gl, acc, xin, u * kChunk * E);
                }
        }
#pragma unroll
        for (int u = 0; u < kQuantUnroll; ++u) cur[u] = nxt[u];
    }
    if constexpr (ERR) {
        // Fix-up pass: only waves that deferred a block's separate non-max sum
        // (rare) read their range again.
        if (p.so.stats && __builtin_amdgcn_readfirstlane(acc.fixup)) {
            for (int i = 0, c = c0; i < n_groups; ++i, c += cstep) {
                Raw<XT> raw[kQuantUnroll];
                load_group32<XT, kQuantUnroll>(raw, p.x, c, c1, ck, lane);
                const QOut o = group_outputs32<B, kQuantUnroll>(p, c, c1, ck);
                const Rsrc xin = group_input32<XT, kQuantUnroll>(p.x, c, c1, ck);
                const int left = c1 - c;
#pragma unroll
                for (int u = 0; u < kQuantUnroll; ++u)
                    if (u < left) {
                        if constexpr (SEARCH)
                            search_chunk<XT, FMT, B, ROT, SUMSQ, kSepFixup>(raw[u], u, o, p, ue, lane,
                                                                            gl, acc);
                        else
                            quantize_chunk<XT, FMT, B, ROT, ERR, SUMSQ, kSepFixup, kPair, ST>(
                                raw[u], u, o, p, ue, lane, gl, acc, xin, u * kChunk * E);
                    }
            }
        }
    }
    if constexpr (AMAX) {
        __shared__ uint32_t s_amax[kWaves];
        const uint32_t wm = wave_max(acc.amax);
        if (lane == 0) s_amax[threadIdx.x / kWave] = wm;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t mm = s_amax[0];
            for (int w = 1; w < kWaves; ++w) mm = max(mm, s_amax[w]);
            p.amax_out[blockIdx.x] = mm;
        }
    }
    if (p.so.stats) {
        // Every lane of a block holds its terms: keep one copy (with pairing,
        // lanes 0 and 1 of each block position hold the two chunks' blocks).
        if (kPair ? gl >= 2 : gl != 0) acc = Acc{};
        write_partial(acc, p.so);
    }
}

template <int XT, int FMT, int B, int ROT, bool ERR, bool SUMSQ, bool SEARCH = false>
__global__ __launch_bounds__(kThreads)
#if FP4Q_QUANT_WPE
__attribute__((amdgpu_waves_per_eu(FP4Q_QUANT_WPE)))
#endif
FP4Q_SGPR_CAP void k_quantize(QParams p) {
    quantize_body<XT, FMT, B, ROT, ERR, SUMSQ, SEARCH, false>(p);
}

// The NVFP4 pass of fp4_quantize_mx_nv (UE4M3, no rotation): k_quantize with
// the nontemporal stores of the batched NVFP4 pass (kBatchNvStore), launched on
// the plain kernel's grid so that its tensor terms are summed in the same
// order as a separate nvfp4_quantize call's.
template <int XT, int B, bool ERR, bool SUMSQ>
__global__ __launch_bounds__(kThreads)
#if FP4Q_QUANT_WPE
__attribute__((amdgpu_waves_per_eu(FP4Q_QUANT_WPE)))
#endif
FP4Q_SGPR_CAP void k_quantize_nv_pair(QParams p) {
    quantize_body<XT, kFmtUe4m3, B, 0, ERR, SUMSQ, false, false, kBatchNvStore>(p);
}

// The MXFP4 pass of fp4_quantize_mx_nv (no rotation): k_quantize plus the
// per-workgroup maxima.  Held to 8 waves per SIMD (64 VGPRs), the occupancy
// of the plain MXFP4 kernel, whose grid it takes (so its tensor terms are
// summed in the same order and match the plain call's bit for bit).
template <int XT, bool ERR, bool SUMSQ>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8)))
FP4Q_SGPR_CAP void k_quantize_amax(QParams p) {
    quantize_body<XT, kFmtMx, 32, 0, ERR, SUMSQ, false, true>(p);
}

// ------------------------------------------------------------ batched launches
// Several tensors in one launch (fp4_quantize_mx_nv_batch): tensor i gets
// workgroups wg_first .. wg_first + wg_count - 1 of the grid and sweeps its
// own chunks with them, exactly as a launch of its own with that grid would.
// Per-workgroup partials and maxima keep their grid-wide slots.
constexpr int kMaxBatch = kMaxBatchTensors;

struct TensorSlot {
    const void* x;
    int64_t n, n_chunks;
    uint8_t* codes;
    uint8_t* scales;
    float* block_mse;
    const float* g_in;  // NVFP4 pass: the tensor's per-tensor scale (device)
    int wg_first, wg_count;
};

struct BatchParams {
    QParams base;  // what the tensors share: format, MSE kind, outputs wanted, slots
    int n;
    TensorSlot t[kMaxBatch];
};

template <int XT, int FMT, int B, bool ERR, bool SUMSQ>
__device__ __forceinline__ void batch_body(const BatchParams& bp) {
    int t = 0;
    while (t + 1 < bp.n && (int)blockIdx.x >= bp.t[t + 1].wg_first) ++t;
    const TensorSlot& s = bp.t[t];
    QParams p = bp.base;
    p.x = s.x;
    p.n = s.n;
    p.n_chunks = s.n_chunks;
    p.n_blocks = s.n / B;
    p.codes = s.codes;
    p.scales = s.scales;
    p.block_mse = s.block_mse;
    p.g_in = s.g_in;
    p.wg_first = s.wg_first;
    p.wg_count = s.wg_count;
    // The NVFP4 pass of a batched combined call stores its outputs with the
    // nontemporal bit (see kBatchNvStore).
    quantize_body<XT, FMT, B, 0, ERR, SUMSQ, false, FMT == kFmtMx,
                  FMT == kFmtMx ? quant_store_policy<FMT>() : kBatchNvStore>(p);
}

// The MXFP4 pass of a batch (per-workgroup maxima for the NVFP4 scales).
template <int XT, bool ERR, bool SUMSQ>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8)))
FP4Q_SGPR_CAP void k_quantize_mx_batch(BatchParams bp) {
    batch_body<XT, kFmtMx, 32, ERR, SUMSQ>(bp);
}

// The NVFP4 pass of a batch (UE4M3 scales under each tensor's given g).
template <int XT, int B, bool ERR, bool SUMSQ>
__global__ __launch_bounds__(kThreads) FP4Q_SGPR_CAP void k_quantize_nv_batch(BatchParams bp) {
    batch_body<XT, kFmtUe4m3, B, ERR, SUMSQ>(bp);
}

// The reductions of a batch, one workgroup per tensor: its tensor terms from
// its workgroups' partials, and (MXFP4 pass) its per-tensor scale from their
// maxima.
struct BatchStats {
    double* partials;
    const uint32_t* amax_part;
    struct {
        void* stats;  // fp4q_stats or NULL
        long long n_blocks;
        float* g_out;  // NULL: no scale to form
        int wg_first, wg_count;
    } t[kMaxBatch];
};

__global__ __launch_bounds__(kThreads) void k_finalize_batch(BatchStats bs) {
    const auto& s = bs.t[blockIdx.x];
    if (s.g_out) {
        const float g = dynamic_g(bs.amax_part + s.wg_first, s.wg_count);
        if (threadIdx.x == 0) *s.g_out = g;
    }
    if (s.stats) {
        StatsOut so{};
        so.partials = bs.partials + s.wg_first;
        so.stats = s.stats;
        so.n_blocks = s.n_blocks;
        sum_partials(so, s.wg_count);
    }
}


// ------------------------------------------------------------ amax pre-pass
struct AParams {
    const void* x;
    int64_t n, n_chunks, cpw;
    uint32_t* part;
    double* sumsq;  // per-workgroup sum x^2 (binary64), written when non-NULL
};

// Max |x| bits of a lane's 8 values (rotated first when ROT != 0); with
// SUMSQ also adds their squares into ss (binary64).
template <int XT, int ROT, bool SUMSQ>
__device__ __forceinline__ uint32_t chunk_absmax_bits(const Raw<XT>& raw, int gl, double& ss) {
    if constexpr (XT == 0 && ROT == 0 && !SUMSQ) {
        const u16x2_t a0 = __builtin_bit_cast(u16x2_t, raw.w.x & 0x7FFF7FFFu);
        const u16x2_t a1 = __builtin_bit_cast(u16x2_t, raw.w.y & 0x7FFF7FFFu);
        const u16x2_t a2 = __builtin_bit_cast(u16x2_t, raw.w.z & 0x7FFF7FFFu);
        const u16x2_t a3 = __builtin_bit_cast(u16x2_t, raw.w.w & 0x7FFF7FFFu);
        const u16x2_t mm = __builtin_elementwise_max(__builtin_elementwise_max(a0, a1),
                                                     __builtin_elementwise_max(a2, a3));
        return (uint32_t)max(mm[0], mm[1]) << 16;
    } else {
        float v[8];
        unpack<XT>(raw, v);
        if constexpr (ROT != 0) rotate8<ROT>(v, gl);
        if constexpr (SUMSQ) {
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = fma((double)v[i], (double)v[i], ss);
        }
        float mf = fmaxf(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))),
                         fmaxf(fmaxf(fabsf(v[4]), fabsf(v[5])), fmaxf(fabsf(v[6]), fabsf(v[7]))));
        return __float_as_uint(mf);
    }
}

template <int XT, int ROT, bool SUMSQ>
__global__ __launch_bounds__(kAmaxThreads) void k_amax(AParams p) {
    __shared__ uint32_t s_m[kAmaxWaves];
    __shared__ double s_ss[kAmaxWaves];
    constexpr int L = ROT ? ROT / kLaneElems : 1;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int gl = lane & (L - 1);
    const WaveRange wr = wave_range<kAmaxWaves, kAmaxUnroll>(p.n_chunks, p.cpw);
    uint32_t mx = 0;
    double ss = 0.0;
    // Elements past the wave's range read as zeros, which leave both the
    // maximum and the sum of squares unchanged.
#if FP4Q_PREFETCH
    Raw<XT> cur[kAmaxUnroll];
    if (wr.n > 0) load_group<XT, kAmaxUnroll>(cur, p.x, p.n, wr.c0, wr.c1, lane);
#endif
    for (int64_t i = 0, c = wr.c0; i < wr.n; ++i, c += wr.step) {
#if FP4Q_PREFETCH
        Raw<XT> nxt[kAmaxUnroll];
        if (i + 1 < wr.n) load_group<XT, kAmaxUnroll>(nxt, p.x, p.n, c + wr.step, wr.c1, lane);
#else
        Raw<XT> cur[kAmaxUnroll];
        load_group<XT, kAmaxUnroll>(cur, p.x, p.n, c, wr.c1, lane);
#endif
        const int64_t left = wr.c1 - c;
#pragma unroll
        for (int u = 0; u < kAmaxUnroll; ++u) {
            if (u < left) {
                double cs = 0.0;
                mx = max(mx, chunk_absmax_bits<XT, ROT, SUMSQ>(cur[u], gl, cs));
                if constexpr (SUMSQ) ss += cs;
            }
        }
#if FP4Q_PREFETCH
#pragma unroll
        for (int u = 0; u < kAmaxUnroll; ++u) cur[u] = nxt[u];
#endif
    }
    mx = wave_max(mx);
    if constexpr (SUMSQ) ss = wave_sum(ss);
    if (lane == 0) {
        s_m[wave] = mx;
        s_ss[wave] = ss;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t m = s_m[0];
        for (int w = 1; w < kAmaxWaves; ++w) m = max(m, s_m[w]);
        p.part[blockIdx.x] = m;
        if constexpr (SUMSQ) {
            double t = 0.0;
            for (int w = 0; w < kAmaxWaves; ++w) t += s_ss[w];
            p.sumsq[blockIdx.x] = t;
        }
    }
}

// ------------------------------------------------------------ per-row scale
// Activations, one token per row: every row is quantized (UE4M3) under its own
// dynamic scale g_r = RN32(amax_r / 2688), 1 when that is 0.  A wave owns whole
// rows (rows w, w + W, ... on a one-round grid): it reads its row once for the
// maximum, builds the row's decode-scale table in its own slice of LDS, then
// reads the row again (now in cache) and quantizes it chunk by chunk exactly as
// k_quantize does.  No workgroup-wide barrier is needed, so waves may own
// different numbers of rows.
struct RowParams {
    QParams q;      // outputs, mse kind and stats of the whole tensor
    int64_t rows, cols;
    float* g_rows;  // rows floats, written
};

// The kUnroll-chunk group starting at chunk k of a row of `cols` elements;
// elements past the row's end read as zeros.
template <int XT>
__device__ __forceinline__ Rsrc row_group_input(const void* xrow, int64_t cols, int64_t k) {
    constexpr int E = XT == 0 ? 2 : 4;
    const int64_t first = k * kChunk;
    int64_t avail = (int64_t)kUnroll * kChunk;
    if (avail > cols - first) avail = cols - first;
    return make_rsrc(static_cast<const char*>(xrow) + first * E, avail * E);
}

template <int XT>
__device__ __forceinline__ void load_row_group(Raw<XT> (&raw)[kUnroll], const void* xrow,
                                               int64_t cols, int64_t k, int lane) {
    constexpr int E = XT == 0 ? 2 : 4;
    const Rsrc r = row_group_input<XT>(xrow, cols, k);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if constexpr (XT == 0) {
            raw[u].w = buf_load16(r, u * kChunk * E + lane * 16);
        } else {
            raw[u].a = buf_load16(r, u * kChunk * E + lane * 32);
            raw[u].b = buf_load16(r, u * kChunk * E + lane * 32 + 16);
        }
    }
}

template <int B>
__device__ __forceinline__ QOut row_outputs(const QParams& p, int64_t row, int64_t cols, int64_t k) {
    const int64_t first = row * cols + k * kChunk;
    int64_t avail = (int64_t)kUnroll * kChunk;
    if (avail > cols - k * kChunk) avail = cols - k * kChunk;
    QOut o;
    o.codes = make_rsrc(p.codes + first / 2, avail / 2);
    o.scales = make_rsrc(p.scales + first / B, avail / B);
    o.mse = make_rsrc(p.block_mse + first / B, p.block_mse ? avail / B * 4 : 0);
    return o;
}

// Wave-local table of the UE4M3 decode scales under g (entries as in
// build_scale_table).  LDS operations of one wave complete in order; the
// wavefront-scope fences keep the compiler from moving the table's accesses
// across the hand-over.
__device__ __forceinline__ void build_wave_table(float4* tab, float g, float D, int lane) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    for (int c = lane; c < 0x7F; c += kWave) {
        const float d = ue_decode((uint32_t)c, kFmtUe4m3) * g;
        const float r = d > 0.0f ? 1.0f / d : 0.0f;
        float lim = -1.0f;
        if (d == 0.0f) lim = __builtin_inff();
        else if (d >= 0x1p-96f && d <= 0x1p100f) lim = d * 4096.0f;
        const bool six = c >= 8 && d >= 0x1p-126f && D >= 0x1p-126f;
        tab[c] = make_float4(d, r, lim, six ? 1.0f : 0.0f);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int XT, int B, int ROT, bool ERR, bool SUMSQ>
__global__ __launch_bounds__(kThreads) void k_quantize_rows(RowParams rp) {
    constexpr int L = B / kLaneElems;
    constexpr int E = XT == 0 ? 2 : 4;
    __shared__ float4 s_tab[kWaves][128];
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int gl = lane & (L - 1);
    const int64_t W = (int64_t)gridDim.x * kWaves;
    const int64_t wid = (int64_t)xcd_slice(blockIdx.x, gridDim.x) * kWaves + wave;
    const int64_t nk = (rp.cols + kChunk - 1) / kChunk;  // chunks per row
    const QParams& p = rp.q;
    float4* tab = s_tab[wave];
    Acc acc;
    for (int64_t row = wid; row < rp.rows; row += W) {
        const char* xrow = static_cast<const char*>(p.x) + row * rp.cols * E;
        // Pass 1: the row's maximum |x| (rotated blocks when rotating).
        uint32_t mx = 0;
        Raw<XT> cur[kUnroll];
        load_row_group<XT>(cur, xrow, rp.cols, 0, lane);
        for (int64_t k = 0; k < nk; k += kUnroll) {
            Raw<XT> nxt[kUnroll];
            if (k + kUnroll < nk) load_row_group<XT>(nxt, xrow, rp.cols, k + kUnroll, lane);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (k + u < nk) {
                    double unused = 0.0;
                    mx = max(mx, chunk_absmax_bits<XT, ROT, false>(cur[u], gl, unused));
                }
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) cur[u] = nxt[u];
        }
        mx = wave_max(mx);
        float g = __uint_as_float(mx) / 2688.0f;
        if (!(g > 0.0f)) g = 1.0f;
        if (lane == 0) rp.g_rows[row] = g;
        UeCtx ue;
        ue.g = g;
        ue.D = 6.0f * g;
        ue.rD = 1.0f / ue.D;
        ue.s_fast_max = (ue.D >= 0x1p-96f && ue.D <= 0x1p100f) ? 4096.0f : -1.0f;
        build_wave_table(tab, g, ue.D, lane);
        ue.tab = tab;
        // Pass 2: quantize the row.
        load_row_group<XT>(cur, xrow, rp.cols, 0, lane);
        for (int64_t k = 0; k < nk; k += kUnroll) {
            Raw<XT> nxt[kUnroll];
            if (k + kUnroll < nk) load_row_group<XT>(nxt, xrow, rp.cols, k + kUnroll, lane);
            const QOut o = row_outputs<B>(p, row, rp.cols, k);
            const Rsrc xin = row_group_input<XT>(xrow, rp.cols, k);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                if (k + u < nk)
                    quantize_chunk<XT, kFmtUe4m3, B, ROT, ERR, SUMSQ>(cur[u], u, o, p, ue, lane, gl, acc,
                                                                      xin, u * kChunk * E);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) cur[u] = nxt[u];
        }
    }
    if (p.so.stats) {
        if (gl != 0) acc = Acc{};
        write_partial(acc, p.so);
    }
}

// Rows of at most kRowChunks * kWaves chunks (8192 elements): one workgroup per
// row, each wave holding up to kRowChunks of the row's chunks (chunks wave,
// wave + 4, ...) in registers, so the row is read from memory once.  The
// row maximum and the decode-scale table go through LDS with workgroup
// barriers, which every wave reaches the same number of times (rows are taken
// per workgroup).  The next row's loads are issued before the current row is
// quantized.
constexpr int kRowChunks = 4;

template <int XT>
__device__ __forceinline__ void load_row_chunks(Raw<XT> (&raw)[kRowChunks], const void* xrow,
                                                int64_t cols, int wave, int lane) {
    constexpr int E = XT == 0 ? 2 : 4;
    const Rsrc r = make_rsrc(xrow, cols * E);
#pragma unroll
    for (int u = 0; u < kRowChunks; ++u) {
        const int off = (u * kWaves + wave) * kChunk * E;  // past the row: zeros
        if constexpr (XT == 0) {
            raw[u].w = buf_load16(r, off + lane * 16);
        } else {
            raw[u].a = buf_load16(r, off + lane * 32);
            raw[u].b = buf_load16(r, off + lane * 32 + 16);
        }
    }
}

template <int XT, int B, int ROT, bool ERR, bool SUMSQ>
__global__ __launch_bounds__(kThreads) void k_quantize_rows_wg(RowParams rp) {
    constexpr int L = B / kLaneElems;
    constexpr int E = XT == 0 ? 2 : 4;
    __shared__ float4 s_tab[kUeCodes];
    __shared__ uint32_t s_m[kWaves];
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int gl = lane & (L - 1);
    const int nk = (int)((rp.cols + kChunk - 1) / kChunk);  // <= kRowChunks * kWaves
    const QParams& p = rp.q;
    const int64_t G = gridDim.x;
    // One row per workgroup: dispatch order; a sweep: XCD-contiguous rows.
    const int64_t first_row = G >= rp.rows ? (int64_t)blockIdx.x : xcd_slice(blockIdx.x, gridDim.x);
    Acc acc;
    Raw<XT> cur[kRowChunks];
    if (first_row < rp.rows)
        load_row_chunks<XT>(cur, static_cast<const char*>(p.x) + first_row * rp.cols * E, rp.cols,
                            wave, lane);
    for (int64_t row = first_row; row < rp.rows; row += G) {
        uint32_t mx = 0;
#pragma unroll
        for (int u = 0; u < kRowChunks; ++u) {
            if (u * kWaves + wave < nk) {
                double unused = 0.0;
                mx = max(mx, chunk_absmax_bits<XT, ROT, false>(cur[u], gl, unused));
            }
        }
        mx = wave_max(mx);
        if (lane == 0) s_m[wave] = mx;
        __syncthreads();  // also: every wave is done with the previous row's table
        uint32_t m = s_m[0];
        for (int w = 1; w < kWaves; ++w) m = max(m, s_m[w]);
        float g = __uint_as_float(m) / 2688.0f;
        if (!(g > 0.0f)) g = 1.0f;
        if (threadIdx.x == 0) rp.g_rows[row] = g;
        UeCtx ue;
        ue.g = g;
        ue.D = 6.0f * g;
        ue.rD = 1.0f / ue.D;
        ue.s_fast_max = (ue.D >= 0x1p-96f && ue.D <= 0x1p100f) ? 4096.0f : -1.0f;
        build_scale_table(s_tab, g, ue.D, kFmtUe4m3);  // ends in a barrier
        ue.tab = s_tab;
        Raw<XT> nxt[kRowChunks];
        if (row + G < rp.rows)
            load_row_chunks<XT>(nxt, static_cast<const char*>(p.x) + (row + G) * rp.cols * E,
                                rp.cols, wave, lane);
#pragma unroll
        for (int u = 0; u < kRowChunks; ++u) {
            const int k = u * kWaves + wave;
            if (k < nk) {
                const int64_t first = row * rp.cols + (int64_t)k * kChunk;
                int64_t avail = rp.cols - (int64_t)k * kChunk;
                if (avail > kChunk) avail = kChunk;
                QOut o;
                o.codes = make_rsrc(p.codes + first / 2, avail / 2);
                o.scales = make_rsrc(p.scales + first / B, avail / B);
                o.mse = make_rsrc(p.block_mse + first / B, p.block_mse ? avail / B * 4 : 0);
                quantize_chunk<XT, kFmtUe4m3, B, ROT, ERR, SUMSQ>(
                    cur[u], 0, o, p, ue, lane, gl, acc,
                    make_rsrc(static_cast<const char*>(p.x) + row * rp.cols * E, rp.cols * E),
                    k * kChunk * E);
            }
        }
#pragma unroll
        for (int u = 0; u < kRowChunks; ++u) cur[u] = nxt[u];
    }
    if (p.so.stats) {
        if (gl != 0) acc = Acc{};
        write_partial(acc, p.so);
    }
}

// Every row of an empty-column tensor gets g = 1.
__global__ void k_fill_ones(float* g, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        g[i] = 1.0f;
}

// ------------------------------------------------------------ dequantize
struct DParams {
    const uint8_t* codes;
    const uint8_t* scales;
    const float* g;
    int fmt;
    int64_t n, n_chunks, cpw;
    void* out;
};

// Stored codes and scales of one chunk group; bytes past the group's valid
// blocks read as zeros (code +0, scale byte 0).
template <int B>
__device__ __forceinline__ void load_codes(const uint8_t* codes, const uint8_t* scales, int64_t n,
                                           int64_t c, int64_t c1, int lane,
                                           uint32_t (&cw)[kUnroll], uint32_t (&sb)[kUnroll]) {
    constexpr int L = B / kLaneElems;
    const int64_t first = c * kChunk;
    int64_t avail = (c1 - c < kUnroll ? c1 - c : kUnroll) * kChunk;
    if (avail > n - first) avail = n - first;
    const Rsrc rc = make_rsrc(codes + first / 2, avail / 2);
    const Rsrc rs = make_rsrc(scales + first / B, avail / B);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        cw[u] = __builtin_amdgcn_raw_buffer_load_b32(rc, (u * kChunk + lane * kLaneElems) / 2, 0, kNt);
        sb[u] = __builtin_amdgcn_raw_buffer_load_b8(rs, u * (kChunk / B) + lane / L, 0, 0);
    }
}

template <int FMT>
__device__ __forceinline__ void dequant_word(uint32_t cw, uint32_t sbyte, int fmt, float g,
                                             float (&xh)[8]) {
    if constexpr (FMT == kFmtMx) {
        decode_word(cw, __uint_as_float(sbyte << 23), xh);
    } else {
        const float d = ue_decode(sbyte, fmt) * g;
        decode_word(cw, 1.0f, xh);
#pragma unroll
        for (int i = 0; i < 8; ++i) xh[i] = xh[i] * d;
    }
}

template <int FMT, int B, int ROT, int OT>
__global__ __launch_bounds__(kThreads) void k_dequant(DParams p) {
    constexpr int L = B / kLaneElems;
    constexpr int E = OT == 1 ? 4 : 2;
    const int lane = threadIdx.x % kWave;
    const int gl = lane & (L - 1);
    const float g = (FMT != kFmtMx && p.g) ? *p.g : 1.0f;
    const WaveRange wr = wave_range(p.n_chunks, p.cpw);
    for (int64_t i = 0, c = wr.c0; i < wr.n; ++i, c += wr.step) {
        uint32_t cw[kUnroll], sb[kUnroll];
        load_codes<B>(p.codes, p.scales, p.n, c, wr.c1, lane, cw, sb);
        const int64_t first = c * kChunk;
        int64_t avail = (wr.c1 - c < kUnroll ? wr.c1 - c : kUnroll) * kChunk;
        if (avail > p.n - first) avail = p.n - first;
        const Rsrc ro = make_rsrc(static_cast<char*>(p.out) + first * E, avail * E);
        const int64_t left = wr.c1 - c;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (u >= left) continue;
            float xh[8];
            dequant_word<FMT>(cw[u], sb[u], p.fmt, g, xh);
            if constexpr (ROT != 0) rotate8<ROT>(xh, gl);
            const int off = (u * kChunk + lane * kLaneElems) * E;
            if constexpr (OT == 1) {
                const u32x4_t a = {__float_as_uint(xh[0]), __float_as_uint(xh[1]),
                                   __float_as_uint(xh[2]), __float_as_uint(xh[3])};
                const u32x4_t b = {__float_as_uint(xh[4]), __float_as_uint(xh[5]),
                                   __float_as_uint(xh[6]), __float_as_uint(xh[7])};
                __builtin_amdgcn_raw_buffer_store_b128(a, ro, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b128(b, ro, off + 16, 0, 0);
            } else {
                uint32_t h[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t b = __float_as_uint(xh[i]);
                    h[i] = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;  // nearest, ties to even
                }
                const u32x4_t w = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                   h[6] | (h[7] << 16)};
                __builtin_amdgcn_raw_buffer_store_b128(w, ro, off, 0, 0);
            }
        }
    }
}

// ------------------------------------------------------------ block MSE of stored codes
struct MParams {
    const void* x;
    const uint8_t* codes;
    const uint8_t* scales;
    const float* g;
    int fmt;
    int64_t n, n_chunks, n_blocks, cpw;
    float* block_mse;
    int mse_kind;
    StatsOut so;
};

// Error terms of one chunk of stored codes (cw) and scale bytes (sb) against
// its values (raw): the same per-element arithmetic and accumulation order as
// quantize_chunk, so the per-block MSE of codes that k_quantize wrote is
// bit-identical to the value it reported.  The max-element term follows the
// lowest index attaining the block maximum, which matters for arbitrary codes.
// SEP: kSepDefer or kSepFixup (see kSepInline).
template <int XT, int FMT, int B, int ROT, bool SUMSQ, int SEP>
__device__ __forceinline__ void mse_chunk(const Raw<XT>& raw, uint32_t cw, uint32_t sb, int u,
                                          Rsrc rm, const MParams& p, float g, int lane, int gl,
                                          Acc& acc) {
    static_assert(SEP != kSepInline, "block MSE defers the separate sums");
    constexpr int L = B / kLaneElems;
    constexpr int kBlocks = kChunk / B;
    float v[8], xh[8];
    unpack<XT>(raw, v);
    if constexpr (ROT != 0) rotate8<ROT>(v, gl);
    dequant_word<FMT>(cw, sb, p.fmt, g, xh);
    float mf = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) mf = fmaxf(mf, fabsf(v[i]));
    const float m = __uint_as_float(group_max<L>(__float_as_uint(mf)));
    double sse = 0.0, ss = 0.0;
    uint32_t key = 0xFFu;  // lowest in-block index attaining m
    float e_key = 0.0f;
    uint32_t any_nz = 0;
#pragma unroll
    for (int i = 7; i >= 0; --i) {
        const float e = v[i] - xh[i];
        if (fabsf(v[i]) == m) {
            key = (uint32_t)(gl * 8 + i);
            e_key = e;
        }
        any_nz |= (xh[i] != 0.0f) ? 1u : 0u;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const double e = (double)(v[i] - xh[i]);
        sse = fma(e, e, sse);
    }
    sse = group_sum<L>(sse);
    if constexpr (SUMSQ) ss = block_sumsq<L, XT == 0 && ROT == 0>(v, __float_as_uint(m));
    any_nz = group_max<L>(any_nz);
#pragma unroll
    for (int s = 1; s < L; s <<= 1) {
        const uint32_t ok = (uint32_t)__shfl_xor((int)key, s);
        const float oe = __shfl_xor(e_key, s);
        if (ok < key) {
            key = ok;
            e_key = oe;
        }
    }
    if (SEP != kSepFixup && p.block_mse) {
        float mse;
        if (p.mse_kind == kMseRel) mse = rel_mse(sse, ss);
        else mse = (float)(sse * (1.0 / B));
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(mse), rm,
                                              gl == 0 ? (u * kBlocks + lane / L) * 4 : kDropped, 0, 0);
    }
    if (p.so.stats) {
        const double mterm = (double)e_key * (double)e_key;
        const bool zero = (m > 0.0f) && !any_nz;
        double nm = sse - mterm;
        const bool sep = needs_separate_sum(zero, sse, nm);
        if constexpr (SEP == kSepDefer) {
            if (sep) nm = 0.0;
            if (__builtin_amdgcn_ballot_w64(sep)) acc.fixup = 1u;
        } else {
            if (__builtin_amdgcn_ballot_w64(sep)) {
                const double s2 = nonmax_sum<L>(v, xh, m, gl);
                if (sep) acc.nonmax += s2;
            }
            return;
        }
        add_block(acc, zero, sse, mterm, nm, ss);
    }
}

// mse_chunk over a wave's range, in mode SEP.
template <int XT, int FMT, int B, int ROT, bool SUMSQ, int SEP>
__device__ __forceinline__ void block_mse_range(const MParams& p, const WaveRange& wr, float g,
                                                int lane, int gl, Acc& acc) {
    for (int64_t i = 0, c = wr.c0; i < wr.n; ++i, c += wr.step) {
        Raw<XT> raw[kUnroll];
        uint32_t cw[kUnroll], sb[kUnroll];
        load_group<XT>(raw, p.x, p.n, c, wr.c1, lane);
        load_codes<B>(p.codes, p.scales, p.n, c, wr.c1, lane, cw, sb);
        const int64_t first = c * kChunk;
        int64_t avail = (wr.c1 - c < kUnroll ? wr.c1 - c : kUnroll) * kChunk;
        if (avail > p.n - first) avail = p.n - first;
        const Rsrc rm = make_rsrc(p.block_mse + first / B, p.block_mse ? avail / B * 4 : 0);
        const int64_t left = wr.c1 - c;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (u < left)
                mse_chunk<XT, FMT, B, ROT, SUMSQ, SEP>(raw[u], cw[u], sb[u], u, rm, p, g, lane, gl, acc);
    }
}

// Block MSE (and tensor terms) of stored codes: the work split of k_quantize,
// chunk by chunk through mse_chunk, with the separate non-max sums deferred
// to a fix-up pass of the waves that need one.
template <int XT, int FMT, int B, int ROT, bool SUMSQ>
__global__ __launch_bounds__(kThreads) FP4Q_SGPR_CAP void k_block_mse(MParams p) {
    constexpr int L = B / kLaneElems;
    const int lane = threadIdx.x % kWave;
    const int gl = lane & (L - 1);
    const float g = (FMT != kFmtMx && p.g) ? *p.g : 1.0f;
    const WaveRange wr = wave_range(p.n_chunks, p.cpw);
    Acc acc;
    block_mse_range<XT, FMT, B, ROT, SUMSQ, kSepDefer>(p, wr, g, lane, gl, acc);
    if (p.so.stats && __builtin_amdgcn_readfirstlane(acc.fixup))
        block_mse_range<XT, FMT, B, ROT, SUMSQ, kSepFixup>(p, wr, g, lane, gl, acc);
    if (p.so.stats) {
        if (gl != 0) acc = Acc{};
        write_partial(acc, p.so);
    }
}

// ------------------------------------------------------------ rotation only
struct RParams {
    const void* x;
    int64_t n, n_chunks, cpw;
    float* out;
};

template <int XT, int ROT>
__global__ __launch_bounds__(kThreads) void k_rotate(RParams p) {
    constexpr int L = ROT / kLaneElems;
    const int lane = threadIdx.x % kWave;
    const int gl = lane & (L - 1);
    const WaveRange wr = wave_range(p.n_chunks, p.cpw);
    for (int64_t i = 0, c = wr.c0; i < wr.n; ++i, c += wr.step) {
        Raw<XT> raw[kUnroll];
        load_group<XT>(raw, p.x, p.n, c, wr.c1, lane);
        const int64_t first = c * kChunk;
        int64_t avail = (wr.c1 - c < kUnroll ? wr.c1 - c : kUnroll) * kChunk;
        if (avail > p.n - first) avail = p.n - first;
        const Rsrc ro = make_rsrc(p.out + first, avail * 4);
        const int64_t left = wr.c1 - c;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (u >= left) continue;
            float v[8];
            unpack<XT>(raw[u], v);
            rotate8<ROT>(v, gl);
            const int off = (u * kChunk + lane * kLaneElems) * 4;
            const u32x4_t a = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                               __float_as_uint(v[3])};
            const u32x4_t b = {__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
                               __float_as_uint(v[7])};
            __builtin_amdgcn_raw_buffer_store_b128(a, ro, off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(b, ro, off + 16, 0, 0);
        }
    }
}

// Empty tensors: zero the stats and/or set g = 1.
__global__ void k_empty(void* stats, float* g_out) {
    if (threadIdx.x != 0) return;
    if (stats) {
        double* s = static_cast<double*>(stats);
        s[0] = s[1] = s[2] = s[3] = 0.0;
        reinterpret_cast<long long*>(s)[4] = 0;
        reinterpret_cast<long long*>(s)[5] = 0;
    }
    if (g_out) *g_out = 1.0f;
}

// ------------------------------------------------------------ host side
int64_t chunks_of(int64_t n) { return (n + kChunk - 1) / kChunk; }

// Workgroups of `kernel` that fit on the current device at once (compute units
// times the occupancy its registers and LDS allow), cached per device and kernel.
int resident_groups(const void* kernel, int threads) {
    struct Entry {
        int dev;
        const void* kernel;
        int groups;
    };
    static std::mutex mu;
    static Entry cache[256];
    static int n_cache = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < n_cache; ++i)
            if (cache[i].dev == dev && cache[i].kernel == kernel) return cache[i].groups;
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
        per_cu <= 0)
        per_cu = 1;
    const int groups = cus * per_cu;
    std::lock_guard<std::mutex> lock(mu);
    if (n_cache < 256) cache[n_cache++] = {dev, kernel, groups};
    return groups;
}

// Grid of a streaming kernel over `chunks` 512-element chunks: one round of
// resident workgroups (so no workgroup waits for a second round), fewer when
// the tensor gives each wave under kMinChunksPerWave chunks.
int grid_for_chunks(int64_t chunks, const void* kernel, int waves = kWaves) {
    int64_t want = (chunks + (int64_t)waves * kMinChunksPerWave - 1) / ((int64_t)waves * kMinChunksPerWave);
    const int64_t cap = (int64_t)resident_groups(kernel, waves * kWave) * kGridRounds;
    if (want > cap) want = cap;
    if (want > kMaxGroups) want = kMaxGroups;
    if (want < 1) want = 1;
    return (int)want;
}

struct Split {
    int G;
    int64_t cpw;
};

// cpw > 0: fixed ranges of `cpw` chunks per wave (short-lived workgroups that
// the dispatcher hands out in order), more per wave where the tensor would
// otherwise need more workgroups than the workspace has partial slots.
// cpw = 0: the balanced one-round split.  cpw < 0: the one-round sweep.
Split split_for(int64_t chunks, const void* kernel, int cpw, int waves = kWaves) {
    if (cpw < 0) return {grid_for_chunks(chunks, kernel, waves), cpw};
    if (cpw > 0) {
        const int64_t min_cpw = (chunks + (int64_t)waves * kMaxGroups - 1) / ((int64_t)waves * kMaxGroups);
        const int64_t c = cpw > min_cpw ? cpw : min_cpw;
        const int64_t G = (chunks + (int64_t)waves * c - 1) / ((int64_t)waves * c);
        return {(int)(G > 0 ? G : 1), c};
    }
    return {grid_for_chunks(chunks, kernel, waves), 0};
}

int report(hipError_t e, const char* what, char* msg, size_t len) {
    if (e == hipSuccess) return 0;
    snprintf(msg, len, "%s: %s", what, hipGetErrorString(e));
    return (int)e;
}

// Sums the partials of a G-workgroup stats kernel.
int launch_finalize(const StatsOut& so, int G, hipStream_t st, char* msg, size_t len) {
    FP4Q_LAUNCH(k_finalize, dim3(1), dim3(kThreads), 0, st, so, G);
    return report(hipGetLastError(), "finalize kernel launch", msg, len);
}

typedef void (*QuantKernel)(QParams);

template <int XT, int FMT, int B, int ROT>
QuantKernel pick_quant(bool err, bool sumsq, bool search, bool amax = false) {
    if constexpr (FMT == kFmtMx && ROT == 0) {
        if (amax) {
            if (!err) return k_quantize_amax<XT, false, false>;
            return sumsq ? k_quantize_amax<XT, true, true> : k_quantize_amax<XT, true, false>;
        }
    }
    if (search) return sumsq ? k_quantize<XT, FMT, B, ROT, true, true, true>
                             : k_quantize<XT, FMT, B, ROT, true, false, true>;
    if (!err) return k_quantize<XT, FMT, B, ROT, false, false>;
    if (!sumsq) return k_quantize<XT, FMT, B, ROT, true, false>;
    return k_quantize<XT, FMT, B, ROT, true, true>;
}

template <int XT, int FMT>
QuantKernel pick_quant_block(int block, int rotate, bool err, bool sumsq, bool search,
                             bool amax = false) {
    if constexpr (FMT == kFmtMx) {
        return rotate ? pick_quant<XT, FMT, 32, 32>(err, sumsq, search)
                      : pick_quant<XT, FMT, 32, 0>(err, sumsq, search, amax);
    } else {
        switch (block) {
            case 8: return pick_quant<XT, FMT, 8, 0>(err, sumsq, search);
            case 16: return rotate ? pick_quant<XT, FMT, 16, 16>(err, sumsq, search)
                                   : pick_quant<XT, FMT, 16, 0>(err, sumsq, search);
            case 32: return rotate ? pick_quant<XT, FMT, 32, 32>(err, sumsq, search)
                                   : pick_quant<XT, FMT, 32, 0>(err, sumsq, search);
            case 64: return pick_quant<XT, FMT, 64, 0>(err, sumsq, search);
            case 128: return pick_quant<XT, FMT, 128, 0>(err, sumsq, search);
            default: return pick_quant<XT, FMT, 256, 0>(err, sumsq, search);
        }
    }
}

template <int XT, int B>
QuantKernel pick_nv_pair(bool err, bool sumsq) {
    if (!err) return k_quantize_nv_pair<XT, B, false, false>;
    return sumsq ? k_quantize_nv_pair<XT, B, true, true> : k_quantize_nv_pair<XT, B, true, false>;
}

template <int XT>
QuantKernel pick_nv_pair_block(int block, bool err, bool sumsq) {
    switch (block) {
        case 8: return pick_nv_pair<XT, 8>(err, sumsq);
        case 16: return pick_nv_pair<XT, 16>(err, sumsq);
        case 32: return pick_nv_pair<XT, 32>(err, sumsq);
        case 64: return pick_nv_pair<XT, 64>(err, sumsq);
        case 128: return pick_nv_pair<XT, 128>(err, sumsq);
        default: return pick_nv_pair<XT, 256>(err, sumsq);
    }
}

typedef void (*RowKernel)(RowParams);

template <int XT, int B, int ROT>
RowKernel pick_rows(bool err, bool sumsq, bool wg) {
    if (wg) {
        if (!err) return k_quantize_rows_wg<XT, B, ROT, false, false>;
        if (!sumsq) return k_quantize_rows_wg<XT, B, ROT, true, false>;
        return k_quantize_rows_wg<XT, B, ROT, true, true>;
    }
    if (!err) return k_quantize_rows<XT, B, ROT, false, false>;
    if (!sumsq) return k_quantize_rows<XT, B, ROT, true, false>;
    return k_quantize_rows<XT, B, ROT, true, true>;
}

template <int XT>
RowKernel pick_rows_block(int block, int rotate, bool err, bool sumsq, bool wg) {
    switch (block) {
        case 8: return pick_rows<XT, 8, 0>(err, sumsq, wg);
        case 16: return rotate ? pick_rows<XT, 16, 16>(err, sumsq, wg) : pick_rows<XT, 16, 0>(err, sumsq, wg);
        case 32: return rotate ? pick_rows<XT, 32, 32>(err, sumsq, wg) : pick_rows<XT, 32, 0>(err, sumsq, wg);
        case 64: return pick_rows<XT, 64, 0>(err, sumsq, wg);
        case 128: return pick_rows<XT, 128, 0>(err, sumsq, wg);
        default: return pick_rows<XT, 256, 0>(err, sumsq, wg);
    }
}

// UE4M3 with one dynamic scale per row (activations): a single kernel, plus the
// finalize kernel when the tensor terms are wanted.
int launch_quantize_rows(const QuantJob& j, char* msg, size_t msg_len) {
    hipStream_t st = static_cast<hipStream_t>(j.stream);
    if (j.n == 0) {
        if (j.rows > 0) {
            FP4Q_LAUNCH(k_fill_ones, dim3(16), dim3(256), 0, st, j.g, j.rows);
            int rc = report(hipGetLastError(), "fill kernel launch", msg, msg_len);
            if (rc) return rc;
        }
        if (j.stats) {
            FP4Q_LAUNCH(k_empty, dim3(1), dim3(64), 0, st, j.stats, nullptr);
            return report(hipGetLastError(), "empty-tensor kernel", msg, msg_len);
        }
        return 0;
    }
    const bool err = (j.block_mse != nullptr) || (j.stats != nullptr);
    const bool rel = (j.block_mse != nullptr && j.mse_kind == kMseRel);
    const bool sumsq = j.stats != nullptr || rel;
    // Rows that fit in the registers of one workgroup take one workgroup each
    // (read once); longer rows are read twice by one wave each.
    const bool wg = (j.cols + kChunk - 1) / kChunk <= (int64_t)kRowChunks * kWaves;
    const RowKernel k = j.xt == 0 ? pick_rows_block<0>(j.block, j.rotate, err, sumsq, wg)
                                  : pick_rows_block<1>(j.block, j.rotate, err, sumsq, wg);
    // One workgroup per row, short-lived, when no stats partials are formed
    // (the dispatcher hands rows out as slots free up: 8192 x 5120 tokens
    // 35.2 -> 32.6 us, 2048 x 5120 11.3 -> 9.4 us); otherwise one round of
    // resident workgroups sweeping the rows.
    int64_t G = wg ? j.rows : (j.rows + kWaves - 1) / kWaves;
    const int64_t cap = resident_groups(reinterpret_cast<const void*>(k), kThreads);
    if (G > cap && !(wg && j.stats == nullptr)) G = cap;
    if (G > kMaxGroups) G = kMaxGroups;
    RowParams rp{};
    QParams& p = rp.q;
    p.x = j.x;
    p.n = j.n;
    p.codes = j.codes;
    p.scales = j.scales;
    p.block_mse = j.block_mse;
    p.mse_kind = j.mse_kind;
    p.fmt = kFmtUe4m3;
    p.so.stats = j.stats;
    p.so.n_blocks = j.n / j.block;
    if (j.ws) p.so.partials = reinterpret_cast<double*>(static_cast<uint8_t*>(j.ws) + kWsPartials);
    rp.rows = j.rows;
    rp.cols = j.cols;
    rp.g_rows = j.g;
    FP4Q_LAUNCH(k, dim3((int)G), dim3(kThreads), 0, st, rp);
    int rc = report(hipGetLastError(), "per-row quantize kernel launch", msg, msg_len);
    if (rc || !j.stats) return rc;
    return launch_finalize(p.so, (int)G, st, msg, msg_len);
}

typedef void (*AmaxKernel)(AParams);

template <bool SUMSQ>
AmaxKernel pick_amax_t(int xt, int rotate) {
    if (xt == 0) {
        if (rotate == 16) return k_amax<0, 16, SUMSQ>;
        if (rotate == 32) return k_amax<0, 32, SUMSQ>;
        return k_amax<0, 0, SUMSQ>;
    }
    if (rotate == 16) return k_amax<1, 16, SUMSQ>;
    if (rotate == 32) return k_amax<1, 32, SUMSQ>;
    return k_amax<1, 0, SUMSQ>;
}

AmaxKernel pick_amax(int xt, int rotate, bool sumsq) {
    return sumsq ? pick_amax_t<true>(xt, rotate) : pick_amax_t<false>(xt, rotate);
}

typedef void (*DequantKernel)(DParams);

template <int FMT, int OT>
DequantKernel pick_dequant_block(int block, int rotate) {
    if constexpr (FMT == kFmtMx) {
        return rotate ? k_dequant<FMT, 32, 32, OT> : k_dequant<FMT, 32, 0, OT>;
    } else {
        switch (block) {
            case 8: return k_dequant<FMT, 8, 0, OT>;
            case 16: return rotate ? k_dequant<FMT, 16, 16, OT> : k_dequant<FMT, 16, 0, OT>;
            case 32: return rotate ? k_dequant<FMT, 32, 32, OT> : k_dequant<FMT, 32, 0, OT>;
            case 64: return k_dequant<FMT, 64, 0, OT>;
            case 128: return k_dequant<FMT, 128, 0, OT>;
            default: return k_dequant<FMT, 256, 0, OT>;
        }
    }
}

typedef void (*MseKernel)(MParams);

template <int XT, int FMT, int B, int ROT>
MseKernel pick_mse(bool sumsq) {
    return sumsq ? k_block_mse<XT, FMT, B, ROT, true> : k_block_mse<XT, FMT, B, ROT, false>;
}

template <int XT, int FMT>
MseKernel pick_mse_block(int block, int rotate, bool sumsq) {
    if constexpr (FMT == kFmtMx) {
        return rotate ? pick_mse<XT, FMT, 32, 32>(sumsq) : pick_mse<XT, FMT, 32, 0>(sumsq);
    } else {
        switch (block) {
            case 8: return pick_mse<XT, FMT, 8, 0>(sumsq);
            case 16: return rotate ? pick_mse<XT, FMT, 16, 16>(sumsq) : pick_mse<XT, FMT, 16, 0>(sumsq);
            case 32: return rotate ? pick_mse<XT, FMT, 32, 32>(sumsq) : pick_mse<XT, FMT, 32, 0>(sumsq);
            case 64: return pick_mse<XT, FMT, 64, 0>(sumsq);
            case 128: return pick_mse<XT, FMT, 128, 0>(sumsq);
            default: return pick_mse<XT, FMT, 256, 0>(sumsq);
        }
    }
}

}  // namespace

namespace {
thread_local void* const* t_events = nullptr;
thread_local int t_pairs = 0;
thread_local int t_used = 0;
}  // namespace

void profile_set(void* const* events, int n_pairs) {
    t_events = n_pairs > 0 ? events : nullptr;
    t_pairs = t_events ? n_pairs : 0;
    t_used = 0;
}

int profile_count() { return t_used; }

void profile_before(void* stream) {
    if (t_used < t_pairs)
        (void)hipEventRecord(static_cast<hipEvent_t>(t_events[2 * t_used]),
                             static_cast<hipStream_t>(stream));
}

void profile_after(void* stream) {
    if (t_used < t_pairs) {
        (void)hipEventRecord(static_cast<hipEvent_t>(t_events[2 * t_used + 1]),
                             static_cast<hipStream_t>(stream));
        ++t_used;
    }
}

int launch_quantize(const QuantJob& j, char* msg, size_t msg_len) {
    if (j.gmode == 3) return launch_quantize_rows(j, msg, msg_len);
    hipStream_t st = static_cast<hipStream_t>(j.stream);
    uint8_t* ws = static_cast<uint8_t*>(j.ws);
    const bool dynamic = (j.fmt != kFmtMx) && (j.gmode == 1);
    if (j.n == 0) {
        if (j.stats || dynamic) {
            FP4Q_LAUNCH(k_empty, dim3(1), dim3(64), 0, st, j.stats, dynamic ? j.g : nullptr);
            return report(hipGetLastError(), "empty-tensor kernel", msg, msg_len);
        }
        return 0;
    }
    const int64_t chunks = chunks_of(j.n);
    QParams p{};
    p.x = j.x;
    p.n = j.n;
    p.n_chunks = chunks;
    p.n_blocks = j.n / j.block;
    p.codes = j.codes;
    p.scales = j.scales;
    p.block_mse = j.block_mse;
    p.mse_kind = j.mse_kind;
    p.fmt = j.fmt;
    p.g_in = nullptr;
    p.so.stats = j.stats;
    p.so.n_blocks = j.n / j.block;
    if (ws) {
        p.so.partials = reinterpret_cast<double*>(ws + kWsPartials);
    }
    const bool err = (j.block_mse != nullptr) || (j.stats != nullptr);
    const bool rel = (j.block_mse != nullptr && j.mse_kind == kMseRel);
    // In the dynamic mode the amax pass reads every element anyway; when sum x^2
    // is wanted only for the tensor stats it is accumulated there, and the
    // quantize kernel skips it.
    const bool sumsq_in_amax = dynamic && j.stats != nullptr && !rel;
    const bool sumsq = (j.stats != nullptr || rel) && !sumsq_in_amax;
    const bool search = j.radius >= 0;
    p.radius = search ? j.radius : 0;
    p.max_byte = j.fmt == kFmtMx ? 254 : (j.fmt == kFmtUe4m3 ? 0x7E : 0xF7);
    QuantKernel k;
    const bool amax = j.amax_out != nullptr;  // MXFP4 pass of fp4_quantize_mx_nv (rotate 0)
    if (j.fmt == kFmtMx)
        k = j.xt == 0 ? pick_quant_block<0, kFmtMx>(32, j.rotate, err, sumsq, search, amax)
                      : pick_quant_block<1, kFmtMx>(32, j.rotate, err, sumsq, search, amax);
    else
        k = j.fmt == kFmtUe4m3
                ? (j.xt == 0 ? pick_quant_block<0, kFmtUe4m3>(j.block, j.rotate, err, sumsq, search)
                             : pick_quant_block<1, kFmtUe4m3>(j.block, j.rotate, err, sumsq, search))
                : (j.xt == 0 ? pick_quant_block<0, kFmtUe5m3>(j.block, j.rotate, err, sumsq, search)
                             : pick_quant_block<1, kFmtUe5m3>(j.block, j.rotate, err, sumsq, search));
    const bool light = j.stats == nullptr && !dynamic && j.fmt != kFmtMx;
    // The amax-writing MXFP4 kernel takes the plain kernel's grid (same occupancy).
    const QuantKernel k_grid =
        !amax ? k
              : (j.xt == 0 ? pick_quant_block<0, kFmtMx>(32, j.rotate, err, sumsq, search)
                           : pick_quant_block<1, kFmtMx>(32, j.rotate, err, sumsq, search));
    if (j.nv_of_pair && j.fmt == kFmtUe4m3 && j.rotate == 0 && !search)
        k = j.xt == 0 ? pick_nv_pair_block<0>(j.block, err, sumsq)
                      : pick_nv_pair_block<1>(j.block, err, sumsq);
    const Split sq = split_for(chunks, reinterpret_cast<const void*>(k_grid),
                               light ? kQuantCpwLight : kQuantCpw);
    const int G = sq.G;
    p.cpw = sq.cpw;
    int G_amax = 0;
    if (j.fmt != kFmtMx && j.gmode != 0) {
        if (dynamic) {
            const AmaxKernel ka = pick_amax(j.xt, j.rotate, sumsq_in_amax);
            const Split sa = split_for(chunks, reinterpret_cast<const void*>(ka),
                                       chunks < kAmaxSmallBelow ? kAmaxCpwSmall : kAmaxCpw, kAmaxWaves);
            AParams a{j.x, j.n, chunks, sa.cpw, reinterpret_cast<uint32_t*>(ws + kWsAmax),
                      sumsq_in_amax ? reinterpret_cast<double*>(ws + kWsAmaxSumsq) : nullptr};
            p.so.sumsq_part = a.sumsq;
            p.so.G_sumsq = sa.G;
            G_amax = sa.G;
            FP4Q_LAUNCH(ka, dim3(G_amax), dim3(kAmaxThreads), 0, st, a);
            int rc = report(hipGetLastError(), "amax kernel launch", msg, msg_len);
            if (rc) return rc;
            p.amax_part = a.part;
            p.n_amax = G_amax;
            p.g_out = j.g;
        } else {
            p.g_in = j.g;
        }
    }
    if (amax) {
        p.amax_out = j.amax_out;
        p.so.amax_part = j.amax_out;
        p.so.n_amax = G;
        p.so.g_out = j.g_from_amax;
    }
    FP4Q_LAUNCH(k, dim3(G), dim3(kThreads), 0, st, p);
    int rc = report(hipGetLastError(), "quantize kernel launch", msg, msg_len);
    if (rc || !(j.stats || amax)) return rc;
    return launch_finalize(p.so, G, st, msg, msg_len);
}

typedef void (*BatchKernel)(BatchParams);

template <int XT>
BatchKernel pick_mx_batch(bool err, bool sumsq) {
    if (!err) return k_quantize_mx_batch<XT, false, false>;
    return sumsq ? k_quantize_mx_batch<XT, true, true> : k_quantize_mx_batch<XT, true, false>;
}

template <int XT, int B>
BatchKernel pick_nv_batch(bool err, bool sumsq) {
    if (!err) return k_quantize_nv_batch<XT, B, false, false>;
    return sumsq ? k_quantize_nv_batch<XT, B, true, true> : k_quantize_nv_batch<XT, B, true, false>;
}

// Splits one pass's grid between the tensors of a batch: each tensor gets the
// workgroups a launch of its own would want (at least kMinChunksPerWave chunks
// per wave), and when their sum exceeds the kernel's resident capacity, that
// capacity in proportion to the tensors' chunks (at least one workgroup for a
// non-empty tensor).  Returns the grid size.
int split_batch(const int64_t* chunks, int n, const void* kernel, TensorSlot* t) {
    const int64_t cap = (int64_t)resident_groups(kernel, kThreads) * kGridRounds;
    int64_t want[kMaxBatch], total_want = 0, total_chunks = 0;
    for (int i = 0; i < n; ++i) {
        want[i] = (chunks[i] + (int64_t)kWaves * kMinChunksPerWave - 1) / ((int64_t)kWaves * kMinChunksPerWave);
        total_want += want[i];
        total_chunks += chunks[i];
    }
    int first = 0;
    for (int i = 0; i < n; ++i) {
        int64_t g = want[i];
        if (total_want > cap && chunks[i] > 0) {
            g = cap * chunks[i] / total_chunks;
            if (g < 1) g = 1;
            if (g > want[i]) g = want[i];
        }
        t[i].wg_first = first;
        t[i].wg_count = (int)g;
        first += (int)g;
    }
    return first;
}

int launch_quantize_mx_nv_batch(const QuantJob* mx, const QuantJob* nv, int n, char* msg,
                                size_t msg_len) {
    hipStream_t st = static_cast<hipStream_t>(nv[0].stream);
    uint8_t* ws = static_cast<uint8_t*>(nv[0].ws);
    const int xt = nv[0].xt, block = nv[0].block;
    // Outputs wanted by any tensor (an empty tensor's block MSE pointer may be NULL).
    bool mx_bm = false, nv_bm = false;
    for (int i = 0; i < n; ++i) {
        mx_bm = mx_bm || mx[i].block_mse != nullptr;
        nv_bm = nv_bm || nv[i].block_mse != nullptr;
    }
    const bool mx_stats = mx[0].stats != nullptr, nv_stats = nv[0].stats != nullptr;
    const bool rel = nv[0].mse_kind == kMseRel;
    const bool mx_err = mx_bm || mx_stats, mx_sumsq = mx_stats || (mx_bm && rel);
    const bool nv_err = nv_bm || nv_stats, nv_sumsq = nv_stats || (nv_bm && rel);
    const BatchKernel kmx = xt == 0 ? pick_mx_batch<0>(mx_err, mx_sumsq) : pick_mx_batch<1>(mx_err, mx_sumsq);
    const BatchKernel knv =
        block == 16 ? (xt == 0 ? pick_nv_batch<0, 16>(nv_err, nv_sumsq) : pick_nv_batch<1, 16>(nv_err, nv_sumsq))
                    : (xt == 0 ? pick_nv_batch<0, 32>(nv_err, nv_sumsq) : pick_nv_batch<1, 32>(nv_err, nv_sumsq));
    int64_t chunks[kMaxBatch];
    for (int i = 0; i < n; ++i) chunks[i] = chunks_of(mx[i].n);

    // MXFP4 pass: quantize, write per-workgroup maxima and partials.
    BatchParams bm{};
    bm.n = n;
    bm.base.mse_kind = mx[0].mse_kind;
    bm.base.fmt = kFmtMx;
    bm.base.max_byte = 254;
    bm.base.cpw = kQuantCpw;
    bm.base.amax_out = reinterpret_cast<uint32_t*>(ws + kWsAmax);
    bm.base.so.partials = reinterpret_cast<double*>(ws + kWsPartials);
    bm.base.so.stats = mx[0].stats;  // a flag here: the per-tensor sums go to each tensor's stats
    for (int i = 0; i < n; ++i)
        bm.t[i] = TensorSlot{mx[i].x, mx[i].n, chunks[i], mx[i].codes, mx[i].scales, mx[i].block_mse,
                             nullptr, 0, 0};
    const int Gm = split_batch(chunks, n, reinterpret_cast<const void*>(kmx), bm.t);
    if (Gm > 0) {
        FP4Q_LAUNCH(kmx, dim3(Gm), dim3(kThreads), 0, st, bm);
        int rc = report(hipGetLastError(), "batched MXFP4 quantize launch", msg, msg_len);
        if (rc) return rc;
    }
    BatchStats fm{};
    fm.partials = bm.base.so.partials;
    fm.amax_part = bm.base.amax_out;
    for (int i = 0; i < n; ++i) {
        fm.t[i].stats = mx[i].stats;
        fm.t[i].n_blocks = mx[i].n / 32;
        fm.t[i].g_out = nv[i].g;
        fm.t[i].wg_first = bm.t[i].wg_first;
        fm.t[i].wg_count = bm.t[i].wg_count;
    }
    FP4Q_LAUNCH(k_finalize_batch, dim3(n), dim3(kThreads), 0, st, fm);
    int rc = report(hipGetLastError(), "batched reduction launch", msg, msg_len);
    if (rc) return rc;

    // NVFP4 pass under the scales the reduction just wrote.
    BatchParams bn{};
    bn.n = n;
    bn.base.mse_kind = nv[0].mse_kind;
    bn.base.fmt = kFmtUe4m3;
    bn.base.max_byte = 0x7E;
    bn.base.cpw = FP4Q_NV_BATCH_CPW;
    bn.base.so.partials = reinterpret_cast<double*>(ws + kWsPartials);
    bn.base.so.stats = nv[0].stats;
    for (int i = 0; i < n; ++i)
        bn.t[i] = TensorSlot{nv[i].x, nv[i].n, chunks[i], nv[i].codes, nv[i].scales, nv[i].block_mse,
                             nv[i].g, 0, 0};
    const int Gn = split_batch(chunks, n, reinterpret_cast<const void*>(knv), bn.t);
    if (Gn > 0) {
        FP4Q_LAUNCH(knv, dim3(Gn), dim3(kThreads), 0, st, bn);
        rc = report(hipGetLastError(), "batched NVFP4 quantize launch", msg, msg_len);
        if (rc) return rc;
    }
    if (!nv[0].stats) return 0;
    BatchStats fn{};
    fn.partials = bn.base.so.partials;
    for (int i = 0; i < n; ++i) {
        fn.t[i].stats = nv[i].stats;
        fn.t[i].n_blocks = nv[i].n / block;
        fn.t[i].wg_first = bn.t[i].wg_first;
        fn.t[i].wg_count = bn.t[i].wg_count;
    }
    FP4Q_LAUNCH(k_finalize_batch, dim3(n), dim3(kThreads), 0, st, fn);
    return report(hipGetLastError(), "batched reduction launch", msg, msg_len);
}

int launch_quantize_mx_nv(const QuantJob& mx, const QuantJob& nv, char* msg, size_t msg_len) {
    if (mx.n == 0) {  // empty: zero stats and g = 1, as the separate calls give
        const int rc = launch_quantize(mx, msg, msg_len);
        return rc ? rc : launch_quantize(nv, msg, msg_len);
    }
    // The MXFP4 pass leaves its per-workgroup maxima in the amax slots of the
    // workspace and its reduction writes g; the NVFP4 pass then reads g as a
    // given scale.  Both reductions run before the next pass in stream order,
    // so the two passes can share the workspace's partial slots.
    QuantJob a = mx;
    a.ws = nv.ws;
    a.amax_out = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(nv.ws) + kWsAmax);
    a.g_from_amax = nv.g;
    int rc = launch_quantize(a, msg, msg_len);
    if (rc) return rc;
    QuantJob b = nv;
    b.gmode = 2;
    b.nv_of_pair = true;
    return launch_quantize(b, msg, msg_len);
}

int launch_dequantize(const DequantJob& j, char* msg, size_t msg_len) {
    if (j.n == 0) return 0;
    hipStream_t st = static_cast<hipStream_t>(j.stream);
    const int64_t chunks = chunks_of(j.n);
    DParams p{j.codes, j.scales, j.g, j.fmt, j.n, chunks, 0, j.out};
    DequantKernel k;
    if (j.fmt == kFmtMx)
        k = j.ot == 1 ? pick_dequant_block<kFmtMx, 1>(32, j.rotate)
                      : pick_dequant_block<kFmtMx, 0>(32, j.rotate);
    else
        k = j.ot == 1 ? pick_dequant_block<kFmtUe4m3, 1>(j.block, j.rotate)
                      : pick_dequant_block<kFmtUe4m3, 0>(j.block, j.rotate);
    const Split sp = split_for(chunks, reinterpret_cast<const void*>(k), kStreamCpwLight);
    p.cpw = sp.cpw;
    FP4Q_LAUNCH(k, dim3(sp.G), dim3(kThreads), 0, st, p);
    return report(hipGetLastError(), "dequantize kernel launch", msg, msg_len);
}

int launch_block_mse(const MseJob& j, char* msg, size_t msg_len) {
    hipStream_t st = static_cast<hipStream_t>(j.stream);
    if (j.n == 0) {
        if (j.stats) {
            FP4Q_LAUNCH(k_empty, dim3(1), dim3(64), 0, st, j.stats, nullptr);
            return report(hipGetLastError(), "empty-tensor kernel", msg, msg_len);
        }
        return 0;
    }
    uint8_t* ws = static_cast<uint8_t*>(j.ws);
    const int64_t chunks = chunks_of(j.n);
    MParams p{};
    p.x = j.x;
    p.codes = j.codes;
    p.scales = j.scales;
    p.g = j.g;
    p.fmt = j.fmt;
    p.n = j.n;
    p.n_chunks = chunks;
    p.n_blocks = j.n / j.block;
    p.block_mse = j.block_mse;
    p.mse_kind = j.mse_kind;
    p.so.stats = j.stats;
    p.so.n_blocks = j.n / j.block;
    if (ws) {
        p.so.partials = reinterpret_cast<double*>(ws + kWsPartials);
    }
    const bool sumsq = (j.stats != nullptr) || (j.mse_kind == kMseRel);
    MseKernel k;
    if (j.fmt == kFmtMx)
        k = j.xt == 0 ? pick_mse_block<0, kFmtMx>(32, j.rotate, sumsq)
                      : pick_mse_block<1, kFmtMx>(32, j.rotate, sumsq);
    else
        k = j.xt == 0 ? pick_mse_block<0, kFmtUe4m3>(j.block, j.rotate, sumsq)
                      : pick_mse_block<1, kFmtUe4m3>(j.block, j.rotate, sumsq);
    const Split sp = split_for(chunks, reinterpret_cast<const void*>(k),
                               j.stats == nullptr ? kStreamCpwLight : kStreamCpw);
    const int G = sp.G;
    p.cpw = sp.cpw;
    FP4Q_LAUNCH(k, dim3(G), dim3(kThreads), 0, st, p);
    int rc = report(hipGetLastError(), "block-mse kernel launch", msg, msg_len);
    if (rc || !j.stats) return rc;
    return launch_finalize(p.so, G, st, msg, msg_len);
}

int launch_rotate(const RotateJob& j, char* msg, size_t msg_len) {
    if (j.n == 0) return 0;
    hipStream_t st = static_cast<hipStream_t>(j.stream);
    const int64_t chunks = chunks_of(j.n);
    RParams p{j.x, j.n, chunks, 0, j.out};
    void (*k)(RParams);
    if (j.xt == 0) k = j.rotate == 16 ? k_rotate<0, 16> : k_rotate<0, 32>;
    else k = j.rotate == 16 ? k_rotate<1, 16> : k_rotate<1, 32>;
    const Split sp = split_for(chunks, reinterpret_cast<const void*>(k), kStreamCpwLight);
    p.cpw = sp.cpw;
    FP4Q_LAUNCH(k, dim3(sp.G), dim3(kThreads), 0, st, p);
    return report(hipGetLastError(), "rotate kernel launch", msg, msg_len);
}

}  // namespace fp4q
