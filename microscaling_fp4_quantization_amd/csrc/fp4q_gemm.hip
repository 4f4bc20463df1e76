// fp4q_gemm.hip -- FP4 GEMMs on gfx950: MXFP4 on the scaled matrix cores,
// NVFP4 on the bf16 matrix cores from operands decoded in LDS or registers.
//
// C (M x N) = A_hat (M x K) * B_hat^T, where A and B are MXFP4 matrices in the
// layout the quantize kernels write: row-major E2M1 codes two per byte (element
// 2j in the low nibble) and one E8M0 scale byte per 32 consecutive elements of
// a row.  For an activation-times-weight product A holds the activations
// (tokens x in-features) and B the weights (out-features x in-features).
//
// The hot loop is v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in E2M1
// (format 4): lane l supplies row l % 32 of its 32 x 64 operand over the
// 32-element K block l / 32, as 16 bytes of packed codes, plus that block's
// scale byte, selected from a 32-bit register by the instruction's byte
// select.  Lane l receives, in register r, row 8 (r / 4) + 4 (l / 32) + r % 4
// and column l % 32 of the 32 x 32 result.  (Fed from LDS at two waves per
// SIMD, as here, this shape sustained 6.3 PFLOP/s on MI355X where the
// 16 x 16 x 128 one sustained 5.4, for the same operand bytes per flop.)
//
// Kernels:
//  k_pack_scales  rewrites each operand's scale bytes (one per 32 elements) into
//                 the order the matrix-core lanes consume them, so that a K
//                 stage's scales for one 32-row operand are one contiguous
//                 256-byte load;
//  k_gemm_mxfp4   a workgroup of 8 waves computes a 256 x 256 tile of C; K
//                 advances 256 at a time through two LDS stages;
//  k_gemm_decode  products of at most 32 rows of A: one pass over B, 32 rows of
//                 B and a range of K per wave (no scale packing);
//  k_gemm_nvfp4   the NVFP4 product (UE4M3 scales per 16, a per-tensor scale
//                 per operand) in the 256 x 256 tiling, each stage decoded to
//                 bf16 in LDS for the bf16 matrix cores;
//  k_gemm_decode_nv  its decode-sized form (k_gemm_decode's units, operands
//                 decoded to bf16 in registers);
//  k_splitk_reduce  adds the binary32 partial products of K ranges when a
//                 product is split along K.
//
// Operand codes go from memory to LDS by direct buffer-to-LDS loads (no
// register staging).  A wave-wide `buffer_load_dwordx4 ... lds` writes its 64
// lanes' 16 bytes to 1 KB of contiguous LDS, lane l at byte 16 l; one such
// load moves 8 rows x 128 bytes, each row one whole cache line (the pattern
// the address units serve fastest: 52 bytes per clock per CU on MI355X,
// against 27 for half lines).  In LDS a stage is row-major, 128 bytes per
// row, with row R's eight 16-byte K blocks stored rotated by R / 2 places, so
// that the 16 lanes served together by one ds_read_b128 hit 16 distinct bank
// groups.
//
// The weight operand B is the instruction's first source and the activations
// A its second, so the result is a tile of C^T: each lane holds runs of 4
// consecutive columns of one row of C.  The finished tile is staged through
// the (then idle) LDS and stored as whole row segments, 16 bytes per lane:
// stores of 32 rows x 16 bytes straight from the accumulators cost about an
// eighth of the GEMM's time at an 8192 x 18944 x 3584 product.
//
// All global accesses are range-checked buffer operations over per-tile
// windows: rows past M or N read zeros (their results are not stored), K
// blocks past K are fetched from an offset past the window (zeros: code +0),
// and stores outside C are dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>

#include "fp4q_launch.h"

namespace fp4q {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef __attribute__((address_space(3))) void* LdsPtr;

constexpr int kWave = 64;
constexpr int kWaves = 8;
constexpr int kThreads = kWave * kWaves;
constexpr int BM = 256, BN = 256;          // workgroup tile: rows of A, rows of B
constexpr int BK = 256;                    // K elements per stage
constexpr int kRowStage = BK / 2;          // code bytes per row per stage (one cache line)
constexpr int kFrag = 32;                  // rows per matrix-core operand
constexpr int WM = 128, WN = 64;           // wave tile: rows of A, rows of B
constexpr int FA = WM / kFrag, FB = WN / kFrag;
constexpr int kLoads = (BM + BN) / 8 / kWaves;  // code loads per wave per stage
constexpr int kPackBytes = 256;            // packed scales per 32-row operand per stage
constexpr int kCodeBytes = (BM + BN) * kRowStage;  // a stage's codes in LDS (64 KB)
constexpr int kScaleBytes = (BM + BN) / kFrag * kPackBytes;  // and its scales (4 KB)
constexpr int kStageBytes = kCodeBytes + kScaleBytes;
constexpr int kEpiBytes = 2 * kCodeBytes;  // LDS the epilogue stages the tile through
constexpr int kFmtE2M1 = 4;                // matrix-core operand format: FP4 E2M1
constexpr int kDropped = (int)0x80000000;  // an offset past every buffer window
constexpr int kPastWindow = 1 << 30;       // every window is at most 2^30 bytes
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy of the stores of C: non-temporal.  C is written once and not
// read back here; cached, it evicts the operand rows the other tiles of the
// XCD are about to read (measured: a fifth of the time of a 8192 x 18944 x
// 3584 product).
constexpr int kStoreNT = 2;
static_assert(BM == BN && kLoads % 2 == 0 && kLoads / 2 * kWaves * 8 == BM, "load plan");
static_assert(BM / kFrag == kWaves, "one scale load per wave per operand");

__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

// ---------------------------------------------------------------------------
// Scale packing.  Operand rows are grouped in 32-row fragments f and K in
// stages s of 256 (8 scale blocks).  Fragment f, stage s owns 256 bytes at
// (f * S + s) * 256: the dword of lane l holds, in byte t, the scale of row
// 32 f + l % 32 and K block 8 s + 2 t + l / 32 -- the block that lane l feeds
// to the instruction of depth t within the stage.  Rows and blocks that do not
// exist get byte 0 (their codes are read as +0, so the product is +0).
//
// One workgroup per (fragment, run of 16 stages): it copies the fragment's
// 32 rows x 128 scale bytes of those stages into LDS (each row's bytes are
// contiguous in memory), then writes the 16 x 256 packed bytes, which are
// contiguous too.  One launch packs both operands: the first workgroups take
// A's fragments, the rest B's.
constexpr int kPackStages = 16;
constexpr int kPackThreads = 256;

struct PackOperand {
    const uint8_t* sc;  // rows x kblocks scale bytes
    int64_t rows;
    int64_t groups;     // workgroups: fragments x runs of stages
    uint32_t* out;      // packed scales
};

__global__ __launch_bounds__(kPackThreads) void k_pack_scales(PackOperand pa, PackOperand pb,
                                                              int64_t kblocks, int64_t stages) {
    __shared__ uint8_t tile[kFrag][kPackStages * 8 + 4];  // padded rows
    const bool second = blockIdx.x >= pa.groups;
    const uint8_t* __restrict__ sc = second ? pb.sc : pa.sc;
    const int64_t rows = second ? pb.rows : pa.rows;
    uint32_t* __restrict__ out = second ? pb.out : pa.out;
    const int64_t g = second ? blockIdx.x - pa.groups : blockIdx.x;
    const int64_t runs = (stages + kPackStages - 1) / kPackStages;
    const int64_t f = g / runs;
    const int64_t s0 = (g % runs) * kPackStages;
    const int t = threadIdx.x;
    // Load: thread t moves row t / 8, bytes 16 (t % 8) .. + 15 of the run.
    {
        const int r = t / 8, c0 = (t % 8) * 16;
        const int64_t row = f * kFrag + r;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const int64_t b = 8 * s0 + c0 + c;
            tile[r][c0 + c] = row < rows && b < kblocks ? sc[row * kblocks + b] : (uint8_t)0;
        }
    }
    __syncthreads();
    // Store: dword d of the run is lane d % 64 of stage s0 + d / 64: row
    // d % 32, bytes of blocks 2 u + (d % 64) / 32, u = 0..3.
    const int n_st = (int)(stages - s0 < kPackStages ? stages - s0 : kPackStages);
    uint32_t* dst = out + (f * stages + s0) * (kPackBytes / 4);
    for (int d = t; d < n_st * 64; d += kPackThreads) {
        const int st = d / 64, lane = d % 64, r = lane % kFrag, h = lane / kFrag;
        const uint8_t* src = &tile[r][st * 8 + h];
        dst[d] = (uint32_t)src[0] | ((uint32_t)src[2] << 8) | ((uint32_t)src[4] << 16) |
                 ((uint32_t)src[6] << 24);
    }
}

// ---------------------------------------------------------------------------
// The GEMM kernel.

struct GParams {
    const uint8_t* a_codes;
    const uint8_t* b_codes;
    const uint8_t* a_pack;  // packed scales of A
    const uint8_t* b_pack;  // packed scales of B
    int64_t M, N, K;
    int64_t S;              // K stages, ceil(K / 256)
    void* c;
    int ct;                 // 0 bf16, 1 f32
    int splits;             // K ranges per tile (1: C directly)
    float* partial;         // splits > 1: binary32 partial products, splits x M x N
};

// Round-to-nearest-even binary32 -> bf16 bits.
__device__ __forceinline__ uint32_t to_bf16(float f) {
    const uint32_t b = __float_as_uint(f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Tile of workgroup g: the 8 XCDs take workgroups round robin, so tiles are
// renumbered to give each XCD a contiguous run, walked in groups of kGroupM
// tile rows so that concurrently running tiles share operand rows in its L2.
constexpr int kGroupM = 4;

__device__ __forceinline__ void tile_of(int64_t g, int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                        int64_t& tn) {
    const int64_t T = tiles_m * tiles_n;
    const int64_t xcd = g % 8, idx = g / 8, per = T / 8, rem = T % 8;
    const int64_t t = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    const int64_t span = (int64_t)kGroupM * tiles_n;
    const int64_t first = (t / span) * kGroupM;
    const int64_t gm = tiles_m - first < kGroupM ? tiles_m - first : kGroupM;
    tm = first + (t % span) % gm;
    tn = (t % span) / gm;
}

// Wait for all of this wave's loads (the next stage's codes and scales) and
// LDS reads, then barrier.  The memory clobber keeps LDS accesses from moving
// across.
__device__ __forceinline__ void wait_all_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N of this wave's loads are in flight, then barrier.  A
// workgroup fence would wait for all of them (the later stage too).  The wait
// is the compiler's builtin, so that it knows the scale registers loaded
// before those N have landed (and adds no wait of its own for them).
template <int N>
__device__ __forceinline__ void wait_loads_barrier() {
    static_assert(N >= 0 && N < 16, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);  // vmcnt(N), expcnt and lgkmcnt unconstrained
    asm volatile("s_barrier" ::: "memory");
}

// Wait for this wave's LDS reads, then barrier: afterwards no wave reads the
// stage buffer any more.  (The compiler's builtin again, so that its own
// bookkeeping of outstanding LDS reads agrees.)
__device__ __forceinline__ void lds_reads_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt unconstrained
    asm volatile("s_barrier" ::: "memory");
}

struct Ops {
    v4i a[FA], b[FB];
};

struct Scales {
    uint32_t a[FA], b[FB];
};

// Scales of a stage from LDS: the packed dwords of the wave's A fragments
// (wm * FA + j) and B fragments (wn * FB + i), lane l's at 4 l.
__device__ __forceinline__ void read_scales(Scales& sc, const uint8_t* stage, int wm, int wn, int lane) {
    const uint8_t* p = stage + kCodeBytes + lane * 4;
#pragma unroll
    for (int j = 0; j < FA; ++j)
        sc.a[j] = *reinterpret_cast<const uint32_t*>(p + (wm * FA + j) * kPackBytes);
#pragma unroll
    for (int i = 0; i < FB; ++i)
        sc.b[i] = *reinterpret_cast<const uint32_t*>(p + (BM / kFrag + wn * FB + i) * kPackBytes);
}

// Operands of depth T within a stage: lane l takes row l % 32 of each
// fragment, K block 2 T + l / 32, stored at position (block + row / 2) % 8.
template <int T>
__device__ __forceinline__ void read_ops(Ops& o, const uint8_t* stage, int a_row, int b_row,
                                         int rot) {
    const int at = ((2 * T + rot) & 7) * 16;
#pragma unroll
    for (int j = 0; j < FA; ++j)
        o.a[j] = *reinterpret_cast<const v4i*>(stage + (a_row + j * kFrag) * kRowStage + at);
#pragma unroll
    for (int i = 0; i < FB; ++i)
        o.b[i] = *reinterpret_cast<const v4i*>(stage + (BM + b_row + i * kFrag) * kRowStage + at);
}

// The 4 instructions of depth T for B fragment I (one per A fragment).
template <int T, int I>
__device__ __forceinline__ void mma_half(v16f (&acc)[FB][FA], const Ops& o, const Scales& sc) {
    const v8i b = v8i{o.b[I][0], o.b[I][1], o.b[I][2], o.b[I][3], 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < FA; ++j) {
        const v8i a = v8i{o.a[j][0], o.a[j][1], o.a[j][2], o.a[j][3], 0, 0, 0, 0};
        acc[I][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            b, a, acc[I][j], kFmtE2M1, kFmtE2M1, T, (int)sc.b[I], T, (int)sc.a[j]);
    }
}

// Four results in the output format: EB = 4 binary32, EB = 2 bf16 (round to
// nearest even), packed in 16 or 8 bytes.
template <int EB>
struct Quad;
template <>
struct Quad<4> {
    typedef u32x4_t T;
    static __device__ __forceinline__ T pack(float a, float b, float c, float d) {
        return u32x4_t{__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
    }
};
// Two binary32 values to bf16 in one v_cvt_pk_bf16_f32, which rounds to
// nearest even as to_bf16 does (for every input but NaN, which stays NaN):
// the epilogue's conversions took about 2 us of a 30 us tile as integer
// arithmetic.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

template <>
struct Quad<2> {
    typedef u32x2_t T;
    static __device__ __forceinline__ T pack(float a, float b, float c, float d) {
        return u32x2_t{pack_bf16x2(a, b), pack_bf16x2(c, d)};
    }
};

// Epilogue through LDS, for rows of C that are whole 16-byte units: the tile
// is written to LDS row-major (in passes of as many rows as 128 KB holds),
// then stored with each lane moving 16 contiguous bytes, so that a store
// covers whole cache lines.  In LDS the 4-column group k of row r sits at
// group k ^ (r % 32): the 32 rows a wave writes at once then fall in distinct
// banks, and a 16-byte read holds the same two groups, possibly swapped.
template <int EB>
__device__ __forceinline__ void store_tile(const v16f (&acc)[FB][FA], uint8_t* lds, Rsrc rc, int wave,
                                           int wm, int wn, int lane, int64_t rows_a, int64_t n0,
                                           int64_t N) {
    constexpr int kPitch = BN * EB;                   // LDS bytes per row
    constexpr int kRowsPass = kEpiBytes / kPitch;     // 256 (bf16) or 128 (f32)
    constexpr int kPasses = BM / kRowsPass;
    constexpr int kRowsInstr = 1024 / kPitch;         // rows per wave-wide 1 KB store
    constexpr int kInstr = kRowsPass / kRowsInstr / kWaves;
    typedef typename Quad<EB>::T QT;
    static_assert(kRowsPass % WM == 0 && kInstr * kRowsInstr * kWaves == kRowsPass, "epilogue plan");
#pragma unroll
    for (int h = 0; h < kPasses; ++h) {
        if (wm * WM / kRowsPass == h) {
#pragma unroll
            for (int j = 0; j < FA; ++j) {
                const int r = wm * WM + j * kFrag + lane % kFrag - h * kRowsPass;
#pragma unroll
                for (int i = 0; i < FB; ++i)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int grp = (wn * WN + i * kFrag + 8 * g) / 4 + lane / kFrag;
                        *reinterpret_cast<QT*>(lds + r * kPitch + (grp ^ (r & 31)) * 4 * EB) =
                            Quad<EB>::pack(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                           acc[i][j][4 * g + 3]);
                    }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int k = 0; k < kInstr; ++k) {
            const int r = (wave * kInstr + k) * kRowsInstr + lane / (kPitch / 16);
            const int q = lane % (kPitch / 16);  // 16-byte unit within the row
            u32x4_t v;
            if (EB == 4) {
                v = *reinterpret_cast<const u32x4_t*>(lds + r * kPitch + ((q ^ (r & 31)) * 16));
            } else {
                const int grp = (2 * q) ^ (r & 31);
                v = *reinterpret_cast<const u32x4_t*>(lds + r * kPitch + (grp >> 1) * 16);
                if (r & 1) v = u32x4_t{v[2], v[3], v[0], v[1]};
            }
            const int64_t row = h * kRowsPass + r, col = n0 + q * (16 / EB);
            const int off = row < rows_a && col < N ? (int)(row * N * EB + col * EB) : kDropped;
            __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, kStoreNT);
        }
        if (h + 1 < kPasses) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
}

// Epilogue straight from the accumulators, element by element (rows of C
// that are not whole 16-byte units).
__device__ __forceinline__ void store_direct(const v16f (&acc)[FB][FA], Rsrc rc, int ct, int wm, int wn,
                                             int lane, int64_t rows_a, int64_t n0, int64_t N) {
    const int eb = ct == 1 ? 4 : 2;
#pragma unroll
    for (int j = 0; j < FA; ++j) {
        const int row = wm * WM + j * kFrag + lane % kFrag;
#pragma unroll
        for (int i = 0; i < FB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t col = n0 + wn * WN + i * kFrag + 8 * (r / 4) + 4 * (lane / kFrag) + r % 4;
                const int off = row < rows_a && col < N ? (int)((row * N + col) * eb) : kDropped;
                if (ct == 1)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), rc, off, 0,
                                                          kStoreNT);
                else
                    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)to_bf16(acc[i][j][r]), rc, off, 0,
                                                          kStoreNT);
            }
    }
}

__global__ __launch_bounds__(kThreads) void k_gemm_mxfp4(GParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kStageBytes];
    // Fetch the epilogue's arguments now: a scalar load still in flight in
    // the K loop would force every LDS-read wait there to drain completely
    // (scalar loads complete out of order on the same counter).
    void* c_ptr = p.c;
    float* partial = p.partial;
    int ct = p.ct;
    asm volatile("" : "+s"(c_ptr), "+s"(partial), "+s"(ct));
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves of 128 x 64
    const int64_t tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    // Workgroup g computes K range `split` of tile g / splits.
    const int splits = p.splits, split = (int)(blockIdx.x % splits);
    int64_t tm, tn;
    tile_of(blockIdx.x / splits, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = tm * BM, n0 = tn * BN;
    const int64_t rows_a = p.M - m0 < BM ? p.M - m0 : BM;
    const int64_t rows_b = p.N - n0 < BN ? p.N - n0 : BN;
    const int rowb = (int)(p.K / 2);
    const Rsrc ra = make_rsrc(p.a_codes + m0 * rowb, rows_a * rowb);
    const Rsrc rb = make_rsrc(p.b_codes + n0 * rowb, rows_b * rowb);
    // Packed scales of this tile's fragments (at most 8 per side).  Every
    // offset below fits 32 bits: K <= 2^23, so S <= 2^15 and a window is at
    // most 2^30 bytes.
    const int K = (int)p.K, S = (int)p.S;
    const int per = (S + splits - 1) / splits;  // stages of each K range
    const int s_lo = split * per, s_hi = s_lo + per < S ? s_lo + per : S;
    const int pack_frag = S * kPackBytes;
    const int64_t fa = (rows_a + kFrag - 1) / kFrag, fb = (rows_b + kFrag - 1) / kFrag;
    const Rsrc rsa = make_rsrc(p.a_pack + (m0 / kFrag) * pack_frag, fa * pack_frag);
    const Rsrc rsb = make_rsrc(p.b_pack + (n0 / kFrag) * pack_frag, fb * pack_frag);

    // Code loads: load q of a wave moves rows 8 d .. 8 d + 7, d = wave + 8 (q
    // % 4), of A (q < 4) or of B; lane l fetches row 8 d + l / 8 into LDS
    // position l % 8 of that row, which holds K block (l % 8 - row / 2) % 8.
    // Since row / 2 = 4 d + l / 16 and d = wave (mod 2), the block is the same
    // for every load of the wave.
    const int blk = ((lane % 8) - 4 * (wave & 1) - lane / 16) & 7;
    const int lane_off = (lane / 8) * rowb + blk * 16;
    // Offset base of this lane's loads for stage s (past K or past this
    // workgroup's K range: an offset past the window, so zeros).
    auto dma_base = [&](int s) {
        const int k0 = s * BK;
        // One compare against a limit that is 0 past the range (a select of
        // the limit, not of the compare, so that no branch splits the loop).
        const int klim = s < s_hi ? K : 0;
        return k0 + blk * 32 < klim ? lane_off + k0 / 2 : kPastWindow;
    };
    auto issue_one = [&](uint8_t* stage, int base, int q) {
        const bool is_a = q < kLoads / 2;
        const int d = wave + kWaves * (q % (kLoads / 2));
        uint8_t* dst = stage + (is_a ? 0 : BM * kRowStage) + d * 8 * kRowStage;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? ra : rb, (LdsPtr)dst, 16, base + 8 * d * rowb,
                                                 0, 0, 0);
    };
    // Scale loads: load r of wave w moves the packed scales of fragment w of
    // A (r = 0) or of B (r = 1) for one stage, 256 contiguous bytes.
    const int sa_off = wave * pack_frag + lane * 4;
    auto scale_base = [&](int s) { return s < s_hi ? s * kPackBytes : kPastWindow; };
    auto issue_scale = [&](uint8_t* stage, int base, int r) {
        uint8_t* dst = stage + kCodeBytes + (r * (BM / kFrag) + wave) * kPackBytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r == 0 ? rsa : rsb, (LdsPtr)dst, 4, sa_off + base, 0,
                                                 0, 0);
    };

    v16f acc[FB][FA];
#pragma unroll
    for (int i = 0; i < FB; ++i)
#pragma unroll
        for (int j = 0; j < FA; ++j) acc[i][j] = v16f{};

    const int a_row = wm * WM + lane % kFrag;  // within the tile
    const int b_row = wn * WN + lane % kFrag;
    const int rot = lane / kFrag + ((lane % kFrag) >> 1);

    // Stage s lives in LDS buffer s % 2 (codes and packed scales).  Each wave
    // moves 10 loads per stage: L0..L7 the code loads q0..q7, L8 and L9 the
    // scale loads of A and B.  Per stage s:
    //  A  wait for stage s (own loads) and barrier;
    //     read the scales and the operands of depths 0 and 1; run depths 0
    //     and 1, reading depths 2 and 3 meanwhile and issuing L5..L9 of stage
    //     s + 1 (every LDS read of stage s is then issued);
    //  B  barrier: buffer s % 2 is free.  Run depths 2 and 3, issuing L0..L4
    //     of stage s + 2 into it.
    // B sits mid-stage so that the stage's LDS reads (about as long as half
    // the stage's matrix work) run beside two depths of instructions, and
    // the loads are spread one or two per 4 instructions, so no wave stalls
    // on a full load queue.  The loads issued after stage s + 1's last one
    // are always L0..L4 of stage s + 2, hence vmcnt(5) at A.  Loads of the
    // two stages past the workgroup's range read zeros.
    auto issue_load = [&](uint8_t* stage, int s, int L) {
        if (L < kLoads) issue_one(stage, dma_base(s), L);
        else issue_scale(stage, scale_base(s), L - kLoads);
    };
    constexpr int kLate = 5;  // loads of a stage issued in the stage before it
#pragma unroll
    for (int L = 0; L < kLoads + 2; ++L) issue_load(lds + (s_lo & 1) * kStageBytes, s_lo, L);
#pragma unroll
    for (int L = 0; L < kLate; ++L) issue_load(lds + ((s_lo + 1) & 1) * kStageBytes, s_lo + 1, L);
    auto step = [&](int s) {
        uint8_t* here = lds + (s & 1) * kStageBytes;
        uint8_t* other = lds + ((s + 1) & 1) * kStageBytes;
        wait_loads_barrier<kLate>();
        Scales sc;
        Ops r0, r1, r2;
        // At most 15 LDS reads in flight (the width of the wait counter).
        read_scales(sc, here, wm, wn, lane);
        __builtin_amdgcn_sched_barrier(0);
        read_ops<0>(r0, here, a_row, b_row, rot);
        __builtin_amdgcn_sched_barrier(0);
        read_ops<1>(r1, here, a_row, b_row, rot);
        __builtin_amdgcn_sched_barrier(0);
        mma_half<0, 0>(acc, r0, sc);
        __builtin_amdgcn_sched_barrier(0);
        issue_load(other, s + 1, 5);
        __builtin_amdgcn_sched_barrier(0);
        mma_half<0, 1>(acc, r0, sc);
        __builtin_amdgcn_sched_barrier(0);
        issue_load(other, s + 1, 6);
        read_ops<2>(r2, here, a_row, b_row, rot);
        read_ops<3>(r0, here, a_row, b_row, rot);
        __builtin_amdgcn_sched_barrier(0);
        mma_half<1, 0>(acc, r1, sc);
        __builtin_amdgcn_sched_barrier(0);
        issue_load(other, s + 1, 7);
        issue_load(other, s + 1, 8);
        __builtin_amdgcn_sched_barrier(0);
        mma_half<1, 1>(acc, r1, sc);
        __builtin_amdgcn_sched_barrier(0);
        issue_load(other, s + 1, 9);
        __builtin_amdgcn_sched_barrier(0);
        lds_reads_barrier();
        mma_half<2, 0>(acc, r2, sc);
        __builtin_amdgcn_sched_barrier(0);
        issue_load(here, s + 2, 0);
        __builtin_amdgcn_sched_barrier(0);
        mma_half<2, 1>(acc, r2, sc);
        __builtin_amdgcn_sched_barrier(0);
        issue_load(here, s + 2, 1);
        __builtin_amdgcn_sched_barrier(0);
        mma_half<3, 0>(acc, r0, sc);
        __builtin_amdgcn_sched_barrier(0);
        issue_load(here, s + 2, 2);
        issue_load(here, s + 2, 3);
        __builtin_amdgcn_sched_barrier(0);
        mma_half<3, 1>(acc, r0, sc);
        __builtin_amdgcn_sched_barrier(0);
        issue_load(here, s + 2, 4);
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int s = s_lo; s < s_hi; ++s) step(s);
    // The zero stages past the range are still landing; LDS is reused below.
    wait_all_barrier();

    if (splits > 1) {
        // Binary32 partial product of this K range, reduced by k_splitk_reduce.
        float* part = partial + (int64_t)split * p.M * p.N;
        const Rsrc rp = make_rsrc(part + m0 * p.N, rows_a * p.N * 4);
        if (((p.N * 4) & 15) == 0) store_tile<4>(acc, lds, rp, wave, wm, wn, lane, rows_a, n0, p.N);
        else store_direct(acc, rp, 1, wm, wn, lane, rows_a, n0, p.N);
        return;
    }

    // Lane l, register r of result (i, j): row m = j * 32 + l % 32 of the wave
    // tile, columns n = i * 32 + 8 (r / 4) + 4 (l / 32) + r % 4.
    const int eb = ct == 1 ? 4 : 2;
    const Rsrc rc = make_rsrc(static_cast<char*>(c_ptr) + m0 * p.N * eb, rows_a * p.N * eb);
    if (((p.N * eb) & 15) == 0) {
        if (ct == 1) store_tile<4>(acc, lds, rc, wave, wm, wn, lane, rows_a, n0, p.N);
        else store_tile<2>(acc, lds, rc, wave, wm, wn, lane, rows_a, n0, p.N);
    } else {
        store_direct(acc, rc, ct, wm, wn, lane, rows_a, n0, p.N);
    }
}

int64_t frags_of(int64_t rows) { return (rows + kFrag - 1) / kFrag; }

// ---------------------------------------------------------------------------
// NVFP4 GEMM.  C = gA gB * (A_v * B_v^T), where A_v and B_v hold each element's
// E2M1 value times its block's UE4M3 scale (blocks of 16 along K) and gA, gB
// are the per-tensor scales.  The matrix cores' block scales are powers of two
// only, and an E2M1 value times a UE4M3 scale (up to 6 significant bits) fits
// neither FP8 nor FP6, but it is exact in bf16: so the operands are decoded
// into bf16 in LDS and multiplied with v_mfma_f32_32x32x16_bf16, and gA gB is
// applied to the binary32 result.
//
// The tile, the waves' 2 x 4 layout and the epilogue are the MXFP4 kernel's.
// K advances 64 per stage through two LDS stages of bf16 (256 + 256 rows x
// 128 bytes).  Each of the 512 threads decodes one row's 64 elements of the
// next stage: two 16-byte code loads and one scale dword into registers, then
// v_cvt_scalef32_pk_f32_fp4 (at scale 1), a binary32 multiply by the block
// scale (v_cvt_f32_fp8 decodes UE4M3 exactly), and the upper halves of the
// exact binary32 products as bf16.  In LDS a row's eight 16-byte pieces are
// rotated by row / 2 as in the MXFP4 kernel; at step j lane l reads piece
// 2 j + l / 32 of row l % 32 of its fragment, for both operands alike.
constexpr int BKN = 64;                        // K elements per NVFP4 stage
constexpr int kNvRow = BKN * 2;                // bf16 bytes per row per stage
constexpr int kNvStage = (BM + BN) * kNvRow;   // 64 KB
static_assert(2 * kNvStage >= kEpiBytes && BM + BN == kThreads, "NVFP4 stage plan");

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float2v __attribute__((ext_vector_type(2)));

struct NvParams {
    const uint8_t* a_codes;
    const uint8_t* a_scales;
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    const float* ga;  // per-tensor scales (device), NULL for 1
    const float* gb;
    int64_t M, N, K;
    void* c;
    int ct;           // 0 bf16, 1 f32
    int splits;       // K ranges per tile (1: C directly)
    float* partial;   // splits > 1: binary32 partial products, splits x M x N
};

// Upper halves of two binary32 values with at most 8 significant bits: their
// bf16 encodings, exactly.
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
    return (__float_as_uint(hi) & 0xFFFF0000u) | (__float_as_uint(lo) >> 16);
}

// Byte i of w as an FP8 E4M3 value in binary32 (exact; UE4M3 scale bytes are
// E4M3 codes with the sign bit clear).  i must fold to a constant.
__device__ __forceinline__ float fp8_byte_f32(uint32_t w, int i) {
    switch (i) {
        case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
        case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
        case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
        default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
    }
}

__global__ __launch_bounds__(kThreads) void k_gemm_nvfp4(NvParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kNvStage];
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = wave >> 2, wn = wave & 3;
    const int64_t tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int splits = p.splits, split = (int)(blockIdx.x % splits);
    int64_t tm, tn;
    tile_of(blockIdx.x / splits, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = tm * BM, n0 = tn * BN;
    const int64_t rows_a = p.M - m0 < BM ? p.M - m0 : BM;
    const int64_t rows_b = p.N - n0 < BN ? p.N - n0 : BN;
    const int rowb = (int)(p.K / 2), kbn = (int)(p.K / 16);
    const int S = (int)(p.K / BKN);
    const int per = (S + splits - 1) / splits;
    const int s_lo = split * per, s_hi = s_lo + per < S ? s_lo + per : S;
    const float gg = (p.ga ? *p.ga : 1.0f) * (p.gb ? *p.gb : 1.0f);

    // Decoding role: waves 0-3 take rows of A, waves 4-7 rows of B (a
    // wave-uniform choice, so each wave has one pair of windows).
    const bool dec_a = wave < BM / kWave;
    const int drow = threadIdx.x - (dec_a ? 0 : BM);
    const Rsrc rcode = dec_a ? make_rsrc(p.a_codes + m0 * rowb, rows_a * rowb)
                             : make_rsrc(p.b_codes + n0 * rowb, rows_b * rowb);
    const Rsrc rscl = dec_a ? make_rsrc(p.a_scales + m0 * kbn, rows_a * kbn)
                            : make_rsrc(p.b_scales + n0 * kbn, rows_b * kbn);
    const int drot = drow / 2;
    auto load = [&](int s, u32x4_t& c0, u32x4_t& c1, uint32_t& sc) {
        const int off = s < s_hi ? drow * rowb + 32 * s : kPastWindow;
        const int soff = s < s_hi ? drow * kbn + 4 * s : kPastWindow;
        c0 = __builtin_amdgcn_raw_buffer_load_b128(rcode, off, 0, 0);
        c1 = __builtin_amdgcn_raw_buffer_load_b128(rcode, off + 16, 0, 0);
        sc = __builtin_amdgcn_raw_buffer_load_b32(rscl, soff, 0, 0);
    };
    auto decode = [&](uint8_t* stage, const u32x4_t& c0, const u32x4_t& c1, uint32_t sc) {
        uint8_t* row = stage + (dec_a ? 0 : BM * kNvRow) + drow * kNvRow;
        float sv[4];
        sv[0] = __builtin_amdgcn_cvt_f32_fp8((int)sc, 0);
        sv[1] = __builtin_amdgcn_cvt_f32_fp8((int)sc, 1);
        sv[2] = __builtin_amdgcn_cvt_f32_fp8((int)sc, 2);
        sv[3] = __builtin_amdgcn_cvt_f32_fp8((int)sc, 3);
#pragma unroll
        for (int pc = 0; pc < 8; ++pc) {
            const uint32_t w = pc < 4 ? c0[pc] : c1[pc - 4];
            const float s = sv[pc / 2];
            float2v f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
            float2v f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
            float2v f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
            float2v f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
            const u32x4_t o = {pack_bf16_exact(f0[0] * s, f0[1] * s), pack_bf16_exact(f1[0] * s, f1[1] * s),
                               pack_bf16_exact(f2[0] * s, f2[1] * s), pack_bf16_exact(f3[0] * s, f3[1] * s)};
            *reinterpret_cast<u32x4_t*>(row + 16 * ((pc + drot) & 7)) = o;
        }
    };

    v16f acc[FB][FA];
#pragma unroll
    for (int i = 0; i < FB; ++i)
#pragma unroll
        for (int j = 0; j < FA; ++j) acc[i][j] = v16f{};

    const int r = lane % kFrag, h = lane / kFrag;
    {
        u32x4_t c0, c1;
        uint32_t sc;
        load(s_lo, c0, c1, sc);
        decode(lds, c0, c1, sc);
    }
    __syncthreads();
    for (int s = s_lo; s < s_hi; ++s) {
        const int cur = (s - s_lo) & 1;
        const uint8_t* st = lds + cur * kNvStage;
        u32x4_t c0, c1;
        uint32_t sc = 0;
        const bool more = s + 1 < s_hi;
        if (more) load(s + 1, c0, c1, sc);
#pragma unroll
        for (int j = 0; j < BKN / 16; ++j) {
            bf16x8_t a[FA], b[FB];
#pragma unroll
            for (int fa = 0; fa < FA; ++fa) {
                const int row = wm * WM + fa * kFrag + r;
                a[fa] = *reinterpret_cast<const bf16x8_t*>(st + row * kNvRow + 16 * ((2 * j + h + row / 2) & 7));
            }
#pragma unroll
            for (int fb = 0; fb < FB; ++fb) {
                const int row = wn * WN + fb * kFrag + r;
                b[fb] = *reinterpret_cast<const bf16x8_t*>(st + BM * kNvRow + row * kNvRow +
                                                           16 * ((2 * j + h + row / 2) & 7));
            }
#pragma unroll
            for (int fb = 0; fb < FB; ++fb)
#pragma unroll
                for (int fa = 0; fa < FA; ++fa)
                    acc[fb][fa] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[fb], a[fa], acc[fb][fa], 0, 0, 0);
        }
        if (more) decode(lds + (cur ^ 1) * kNvStage, c0, c1, sc);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < FB; ++i)
#pragma unroll
        for (int j = 0; j < FA; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] *= gg;

    if (splits > 1) {
        float* part = p.partial + (int64_t)split * p.M * p.N;
        const Rsrc rp = make_rsrc(part + m0 * p.N, rows_a * p.N * 4);
        if (((p.N * 4) & 15) == 0) store_tile<4>(acc, lds, rp, wave, wm, wn, lane, rows_a, n0, p.N);
        else store_direct(acc, rp, 1, wm, wn, lane, rows_a, n0, p.N);
        return;
    }
    const int eb = p.ct == 1 ? 4 : 2;
    const Rsrc rc = make_rsrc(static_cast<char*>(p.c) + m0 * p.N * eb, rows_a * p.N * eb);
    if (((p.N * eb) & 15) == 0) {
        if (p.ct == 1) store_tile<4>(acc, lds, rc, wave, wm, wn, lane, rows_a, n0, p.N);
        else store_tile<2>(acc, lds, rc, wave, wm, wn, lane, rows_a, n0, p.N);
    } else {
        store_direct(acc, rc, p.ct, wm, wn, lane, rows_a, n0, p.N);
    }
}


// ---------------------------------------------------------------------------
// Decode-sized products: M <= 32 rows of A (a batch of tokens), any N and K.
// The product is a pass over B, so the work is cut into units of one 32-row
// fragment of B and one range of K segments (256 elements each), one unit per
// wave; the waves of a workgroup (4, or 1 when A has more than 8 rows) share
// nothing but the launch.  A unit
// streams its segments through three LDS buffers of its own (two segments in
// flight while the third is read): B's 32 rows and A's rows (8 AR of them,
// AR = ceil(M / 8); the others read a zero slot) by direct buffer-to-LDS
// loads, 8 rows x 128 bytes per instruction, rotated as in the tile kernel,
// and each operand's 32 rows x 8 scale bytes by one dword-wide direct load
// (so the scale rows must start on 4-byte boundaries: K a multiple of 128 and
// both scale arrays 4-byte aligned; other shapes take the tile kernel).
//
// Within a segment the instruction of depth t takes from lane l (row l % 32,
// half h = l / 32) the 16 bytes 64 h + 16 t of the row's 128, i.e. the
// 32-element block 4 h + t of the segment, for both operands alike: every
// K block meets its partner once, so the sum is the same dot product, and a
// lane's four scale bytes for the segment are consecutive (one LDS dword,
// byte t for depth t).
//
// A unit ends with a 32 x 32 binary32 tile (rows of B by rows of A).  With
// one K range per fragment it is C; otherwise it is the range's partial
// product, and k_splitk_reduce adds the ranges in binary64 and rounds once.
#ifndef FP4Q_DEC_BUFS
#define FP4Q_DEC_BUFS 3
#endif
constexpr int kDecBufs = FP4Q_DEC_BUFS;    // LDS buffers per unit
// Units (waves) per workgroup: 4 for one row group of A, else 1.  Measured
// (Qwen2.5-7B projections, 1 / 16 / 32 tokens): one-wave workgroups spread
// the units over more CUs and won 0.1-1.5 us at 16 and 32 tokens, but lost
// 1.1 us at 1 token x 3584 x 18944.
constexpr int dec_waves(int ar) { return ar == 1 ? 4 : 1; }
constexpr int kDecMaxM = 32;

template <int AR>
struct DecLayout {
    static constexpr int kB = kFrag * kRowStage;       // B codes, 4 KB
    static constexpr int kA = AR * 8 * kRowStage;      // A codes
    static constexpr int kBs = kFrag * 8;              // B scale bytes
    static constexpr int kAs = kFrag * 8;              // A scale bytes
    static constexpr int kBuf = kB + kA + kBs + kAs;
    static constexpr int kZero = kDecBufs * kBuf;      // 16 zero bytes
    static constexpr int kUnit = kZero + 16;
    static constexpr int kLoads = 4 + AR + 2;          // direct loads per segment
    static_assert(kBuf % 16 == 0 && (kDecBufs - 1) * kLoads < 64, "decode layout");
};

struct DecParams {
    const uint8_t* a_codes;
    const uint8_t* a_scales;
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    int64_t M, N, K;
    int S;           // K segments, ceil(K / 256)
    int splits;      // K ranges per fragment
    int64_t units;   // fragments of B x splits
    void* c;         // splits == 1
    int ct;          // 0 bf16, 1 f32
    float* partial;  // splits > 1: splits x M x N binary32
};

// s_waitcnt vmcnt(N) for N < 64 (the count's high bits sit at bits 14-15),
// expcnt and lgkmcnt unconstrained.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Depth T of a segment: scale byte T of each lane's dword.
template <int T>
__device__ __forceinline__ v16f mma_dec(v16f acc, v4i b, v4i a, int sb, int sa) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v8i{b[0], b[1], b[2], b[3], 0, 0, 0, 0},
                                                           v8i{a[0], a[1], a[2], a[3], 0, 0, 0, 0}, acc,
                                                           kFmtE2M1, kFmtE2M1, T, sb, T, sa);
}

template <int AR, int W>
__global__ __launch_bounds__(W * kWave) void k_gemm_decode(DecParams p) {
    typedef DecLayout<AR> L;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[W * L::kUnit];
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t unit = (int64_t)blockIdx.x * W + wave;
    if (unit >= p.units) return;  // the whole wave; no workgroup barrier follows
    const int splits = p.splits, split = (int)(unit % splits);
    const int64_t n0 = unit / splits * kFrag;
    const int64_t rows_b = p.N - n0 < kFrag ? p.N - n0 : kFrag;
    const int rowb = (int)(p.K / 2), kb = (int)(p.K / 32), S = p.S;
    const int per = (S + splits - 1) / splits;
    const int s_lo = split * per, s_hi = s_lo + per < S ? s_lo + per : S;
    // Windows: this fragment's rows of B, all M rows of A (rows past them read
    // zeros).  Every offset fits 32 bits: K <= 2^23 and at most 32 rows.
    const Rsrc rb = make_rsrc(p.b_codes + n0 * rowb, rows_b * rowb);
    const Rsrc ra = make_rsrc(p.a_codes, p.M * rowb);
    const Rsrc rbs = make_rsrc(p.b_scales + n0 * kb, rows_b * kb);
    const Rsrc ras = make_rsrc(p.a_scales, p.M * kb);
    uint8_t* base = lds + wave * L::kUnit;
    *reinterpret_cast<u32x4_t*>(base + L::kZero) = u32x4_t{0u, 0u, 0u, 0u};  // lanes write the same zeros

    // Direct loads.  Code instruction q moves rows 8 q .. 8 q + 7: lane l
    // fetches row 8 q + l / 8 into LDS slot l % 8 of that row, which holds
    // the row's 16-byte piece (l % 8 - row / 2) mod 8; row / 2 = 4 q + l / 16.
    // The scale instruction of an operand moves its 32 rows' 8 bytes of the
    // segment, dword l % 2 of row l / 2 per lane.  Pieces and blocks past K
    // (or segments past the unit's range) take an offset past the window:
    // zeros.
    const int crow = lane / 8, cslot = lane % 8;
    auto issue = [&](int s, uint8_t* buf) {
        const int klim = s < s_hi ? rowb : 0;
        const int slim = s < s_hi ? kb : 0;
#pragma unroll
        for (int q = 0; q < 4 + AR; ++q) {
            const bool is_b = q < 4;
            const int qq = is_b ? q : q - 4;
            const int piece = (cslot - 4 * (qq & 1) - lane / 16) & 7;
            const int pos = 128 * s + 16 * piece;
            const int off = pos < klim ? (8 * qq + crow) * rowb + pos : kDropped;
            uint8_t* dst = buf + (is_b ? 0 : L::kB) + qq * 8 * kRowStage;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(is_b ? rb : ra, (LdsPtr)dst, 16, off, 0, 0, 0);
        }
        const int spos = 8 * s + 4 * (lane % 2);
        const int soff = spos < slim ? (lane / 2) * kb + spos : kDropped;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rbs, (LdsPtr)(buf + L::kB + L::kA), 4, soff, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ras, (LdsPtr)(buf + L::kB + L::kA + L::kBs), 4, soff, 0, 0, 0);
    };

    // Reads: lane l takes row r = l % 32, half h = l / 32; depth t's piece
    // 4 h + t sits in slot (4 h + t + r / 2) mod 8.  A rows past 8 AR read the
    // zero slot.
    const int r = lane % kFrag, h = lane / kFrag;
    const bool a_real = r < 8 * AR;
    constexpr int kAhead = kDecBufs - 1;  // segments in flight while one is read
    v16f acc = {};
#pragma unroll
    for (int i = 0; i < kAhead; ++i) issue(s_lo + i, base + i * L::kBuf);
    int cur = 0;
    for (int s = s_lo; s < s_hi; ++s) {
        const int nxt = cur == 0 ? kAhead : cur - 1;  // (cur + kAhead) mod kDecBufs
        issue(s + kAhead, base + nxt * L::kBuf);
        wait_vm<kAhead * L::kLoads>();
        __builtin_amdgcn_sched_barrier(0);
        const uint8_t* buf = base + cur * L::kBuf;
        v4i bo[4], ao[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int slot = (4 * h + t + r / 2) & 7;
            bo[t] = *reinterpret_cast<const v4i*>(buf + r * kRowStage + 16 * slot);
            ao[t] = *reinterpret_cast<const v4i*>(a_real ? buf + L::kB + r * kRowStage + 16 * slot
                                                         : base + L::kZero);
        }
        const int sb = *reinterpret_cast<const int*>(buf + L::kB + L::kA + r * 8 + 4 * h);
        const int sa = *reinterpret_cast<const int*>(buf + L::kB + L::kA + L::kBs + r * 8 + 4 * h);
        acc = mma_dec<0>(acc, bo[0], ao[0], sb, sa);
        acc = mma_dec<1>(acc, bo[1], ao[1], sb, sa);
        acc = mma_dec<2>(acc, bo[2], ao[2], sb, sa);
        acc = mma_dec<3>(acc, bo[3], ao[3], sb, sa);
        __builtin_amdgcn_sched_barrier(0);
        cur = cur == kAhead ? 0 : cur + 1;
    }
    wait_vm<0>();  // the trailing (empty) loads, before the wave's LDS is left

    // Register e of lane l: row of B 8 (e / 4) + 4 h + e % 4, row of A l % 32.
    const int64_t m = lane % kFrag;
    if (splits == 1) {
        const int eb = p.ct == 1 ? 4 : 2;
        const Rsrc rc = make_rsrc(p.c, p.M * p.N * eb);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t n = n0 + 8 * (e / 4) + 4 * h + e % 4;
            const int off = m < p.M && n < p.N ? (int)((m * p.N + n) * eb) : kDropped;
            if (p.ct == 1)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[e]), rc, off, 0, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b16((unsigned short)to_bf16(acc[e]), rc, off, 0, 0);
        }
    } else {
        const Rsrc rp = make_rsrc(p.partial + split * p.M * p.N, p.M * p.N * 4);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t n = n0 + 8 * (e / 4) + 4 * h + e % 4;
            const int off = m < p.M && n < p.N ? (int)((m * p.N + n) * 4) : kDropped;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[e]), rp, off, 0, 0);
        }
    }
}


// NVFP4 decode kernel (M <= 32): the units, buffers and direct loads of
// k_gemm_decode, with each operand's 32 rows x 16 UE4M3 scale bytes of a
// segment brought in by two dword-wide direct loads, and the arithmetic of
// k_gemm_nvfp4: within a segment lane l (row l % 32, half h = l / 32) reads
// the 16-byte pieces 4 h + i (i = 0..3) of its row; bytes 4 t .. 4 t + 3 of
// piece i are the 8 elements it feeds to bf16 step 4 i + t, decoded in
// registers to v * s_hat with their block's scale (block 8 h + 2 i + t / 2 of
// the segment: the lane's scale bytes are one 8-byte LDS read).  A and B are
// read and paired alike, so every element meets its partner once.
template <int AR>
struct NvDecLayout {
    static constexpr int kB = kFrag * kRowStage;       // B codes, 4 KB
    static constexpr int kA = AR * 8 * kRowStage;      // A codes
    static constexpr int kS = kFrag * 16;              // scale bytes per operand
    static constexpr int kBuf = kB + kA + 2 * kS;
    static constexpr int kZero = kDecBufs * kBuf;
    static constexpr int kUnit = kZero + 16;
    static constexpr int kLoads = 4 + AR + 2 + 2;
    static_assert(kBuf % 16 == 0 && (kDecBufs - 1) * kLoads < 64, "nvfp4 decode layout");
};

struct NvDecParams {
    const uint8_t* a_codes;
    const uint8_t* a_scales;
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    const float* ga;
    const float* gb;
    int64_t M, N, K;
    int S;           // K segments, ceil(K / 256)
    int splits;
    int64_t units;
    void* c;
    int ct;
    float* partial;
};

// 8 elements (one dword of codes) as bf16, times a block scale: exact.
__device__ __forceinline__ bf16x8_t decode8_bf16(uint32_t w, float s) {
    const float2v f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const float2v f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const float2v f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const float2v f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    const u32x4_t o = {pack_bf16_exact(f0[0] * s, f0[1] * s), pack_bf16_exact(f1[0] * s, f1[1] * s),
                       pack_bf16_exact(f2[0] * s, f2[1] * s), pack_bf16_exact(f3[0] * s, f3[1] * s)};
    return __builtin_bit_cast(bf16x8_t, o);
}

template <int AR, int W>
__global__ __launch_bounds__(W * kWave) void k_gemm_decode_nv(NvDecParams p) {
    typedef NvDecLayout<AR> L;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[W * L::kUnit];
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t unit = (int64_t)blockIdx.x * W + wave;
    if (unit >= p.units) return;  // the whole wave; no workgroup barrier follows
    const int splits = p.splits, split = (int)(unit % splits);
    const int64_t n0 = unit / splits * kFrag;
    const int64_t rows_b = p.N - n0 < kFrag ? p.N - n0 : kFrag;
    const int rowb = (int)(p.K / 2), kbn = (int)(p.K / 16), S = p.S;
    const int per = (S + splits - 1) / splits;
    const int s_lo = split * per, s_hi = s_lo + per < S ? s_lo + per : S;
    const float gg = (p.ga ? *p.ga : 1.0f) * (p.gb ? *p.gb : 1.0f);
    const Rsrc rb = make_rsrc(p.b_codes + n0 * rowb, rows_b * rowb);
    const Rsrc ra = make_rsrc(p.a_codes, p.M * rowb);
    const Rsrc rbs = make_rsrc(p.b_scales + n0 * kbn, rows_b * kbn);
    const Rsrc ras = make_rsrc(p.a_scales, p.M * kbn);
    uint8_t* base = lds + wave * L::kUnit;
    *reinterpret_cast<u32x4_t*>(base + L::kZero) = u32x4_t{0u, 0u, 0u, 0u};

    const int crow = lane / 8, cslot = lane % 8;
    auto issue = [&](int s, uint8_t* buf) {
        const int klim = s < s_hi ? rowb : 0;
        const int slim = s < s_hi ? kbn : 0;
#pragma unroll
        for (int q = 0; q < 4 + AR; ++q) {
            const bool is_b = q < 4;
            const int qq = is_b ? q : q - 4;
            const int piece = (cslot - 4 * (qq & 1) - lane / 16) & 7;
            const int pos = 128 * s + 16 * piece;
            const int off = pos < klim ? (8 * qq + crow) * rowb + pos : kDropped;
            uint8_t* dst = buf + (is_b ? 0 : L::kB) + qq * 8 * kRowStage;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(is_b ? rb : ra, (LdsPtr)dst, 16, off, 0, 0, 0);
        }
        // Scales: instruction q moves rows 16 q .. 16 q + 15, dword lane % 4 of
        // row 16 q + lane / 4.
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int spos = 16 * s + 4 * (lane % 4);
            const int soff = spos < slim ? (16 * q + lane / 4) * kbn + spos : kDropped;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rbs, (LdsPtr)(buf + L::kB + L::kA + q * 256), 4, soff, 0,
                                                     0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ras, (LdsPtr)(buf + L::kB + L::kA + L::kS + q * 256), 4,
                                                     soff, 0, 0, 0);
        }
    };

    const int r = lane % kFrag, h = lane / kFrag;
    const bool a_real = r < 8 * AR;
    constexpr int kAhead = kDecBufs - 1;
    v16f acc = {};
#pragma unroll
    for (int i = 0; i < kAhead; ++i) issue(s_lo + i, base + i * L::kBuf);
    int cur = 0;
    for (int s = s_lo; s < s_hi; ++s) {
        const int nxt = cur == 0 ? kAhead : cur - 1;
        issue(s + kAhead, base + nxt * L::kBuf);
        wait_vm<kAhead * L::kLoads>();
        __builtin_amdgcn_sched_barrier(0);
        const uint8_t* buf = base + cur * L::kBuf;
        const u32x2_t sbw = *reinterpret_cast<const u32x2_t*>(buf + L::kB + L::kA + r * 16 + 8 * h);
        const u32x2_t saw = *reinterpret_cast<const u32x2_t*>(buf + L::kB + L::kA + L::kS + r * 16 + 8 * h);
        u32x4_t bo[4], ao[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int slot = (4 * h + i + r / 2) & 7;
            bo[i] = *reinterpret_cast<const u32x4_t*>(buf + r * kRowStage + 16 * slot);
            ao[i] = *reinterpret_cast<const u32x4_t*>(a_real ? buf + L::kB + r * kRowStage + 16 * slot
                                                             : base + L::kZero);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int blk = 2 * i + t / 2;  // scale byte of the lane's 8
                const float sb = fp8_byte_f32(sbw[blk / 4], blk % 4);
                const float sa = fp8_byte_f32(saw[blk / 4], blk % 4);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(decode8_bf16(bo[i][t], sb),
                                                              decode8_bf16(ao[i][t], sa), acc, 0, 0, 0);
            }
        __builtin_amdgcn_sched_barrier(0);
        cur = cur == kAhead ? 0 : cur + 1;
    }
    wait_vm<0>();

#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] *= gg;
    const int64_t m = lane % kFrag;
    if (splits == 1) {
        const int eb = p.ct == 1 ? 4 : 2;
        const Rsrc rc = make_rsrc(p.c, p.M * p.N * eb);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t n = n0 + 8 * (e / 4) + 4 * h + e % 4;
            const int off = m < p.M && n < p.N ? (int)((m * p.N + n) * eb) : kDropped;
            if (p.ct == 1)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[e]), rc, off, 0, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b16((unsigned short)to_bf16(acc[e]), rc, off, 0, 0);
        }
    } else {
        const Rsrc rp = make_rsrc(p.partial + split * p.M * p.N, p.M * p.N * 4);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t n = n0 + 8 * (e / 4) + 4 * h + e % 4;
            const int off = m < p.M && n < p.N ? (int)((m * p.N + n) * 4) : kDropped;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[e]), rp, off, 0, 0);
        }
    }
}

// C = sum over the K ranges of their binary32 partial products, added in
// binary64 in range order and rounded once to binary32 (then to bf16 for a
// bf16 C): one rounding more than the accumulation's own, the same for every
// run.  Four elements per thread, grid-stride.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ partial, int splits,
                                                       int64_t count, void* c, int ct) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
    for (int64_t e0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; e0 < count; e0 += stride) {
        const int n = count - e0 < 4 ? (int)(count - e0) : 4;
        double s[4] = {0.0, 0.0, 0.0, 0.0};
        if (n == 4 && (count & 3) == 0) {
            // Groups of 8 ranges: their loads issue together, the adds stay
            // in range order.
            for (int i0 = 0; i0 < splits; i0 += 8) {
                float4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (i0 + u < splits)
                        v[u] = *reinterpret_cast<const float4*>(partial + (int64_t)(i0 + u) * count + e0);
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (i0 + u < splits) {
                        s[0] += v[u].x;
                        s[1] += v[u].y;
                        s[2] += v[u].z;
                        s[3] += v[u].w;
                    }
            }
        } else {
            for (int i = 0; i < splits; ++i)
                for (int q = 0; q < n; ++q) s[q] += partial[(int64_t)i * count + e0 + q];
        }
        for (int q = 0; q < n; ++q) {
            const float f = (float)s[q];
            if (ct == 1) static_cast<float*>(c)[e0 + q] = f;
            else static_cast<uint16_t*>(c)[e0 + q] = (uint16_t)to_bf16(f);
        }
    }
}

// K ranges per tile.  When the tiles alone fill less than two waves of
// workgroups over the chip (256 CUs, one workgroup each), K is split so that
// the modelled time -- rounds of workgroups x (stages per range + 2 for the
// prologue and epilogue), plus the partial products' round trip through
// memory -- is least.  A function of the shape only, so that the workspace
// size is too.
constexpr int kChipGroups = 256;
constexpr double kStageBytes_Mem = 6.75e6;   // bytes of memory traffic in one stage's time
constexpr int64_t kMaxPartialBytes = (int64_t)1 << 28;

int splits_for(int64_t M, int64_t N, int64_t K) {
    const int64_t S = (K + BK - 1) / BK;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    if (S < 2 || tiles >= 2 * kChipGroups || N * 4 >= ((int64_t)1 << 23)) return 1;
    auto cost = [&](int64_t sp) {
        const int64_t per = (S + sp - 1) / sp;
        const int64_t rounds = (tiles * sp + kChipGroups - 1) / kChipGroups;
        return (double)(rounds * (per + 2)) + (sp > 1 ? (double)sp * M * N * 8 / kStageBytes_Mem : 0.0);
    };
    int64_t best = 1;
    double best_cost = cost(1);
    for (int64_t sp = 2; sp <= S && sp <= 64; ++sp) {
        const int64_t per = (S + sp - 1) / sp;
        const int64_t eff = (S + per - 1) / per;  // ranges that are not empty
        if (eff != sp || sp * M * N * 4 > kMaxPartialBytes) continue;
        const double c = cost(sp);
        if (c < best_cost) {
            best_cost = c;
            best = sp;
        }
    }
    return (int)best;
}

int64_t packed_bytes(int64_t M, int64_t N, int64_t K) {
    return (frags_of(M) + frags_of(N)) * ((K + BK - 1) / BK) * kPackBytes;
}

// The decode kernel takes products of at most 32 rows of A whose scale rows
// start on 4-byte boundaries.  Its K ranges per fragment of B: one (C is
// written directly) when the fragments alone give half of kDecUnits units;
// else enough for about kDecUnits units, each range at least two segments,
// all ranges non-empty, the partials within kMaxPartialBytes.  The reduction
// is a second launch, which costs about as much as doubling the units gains
// (measured on Qwen2.5-7B projections: 18944 x 3584 weights are fastest
// with 592 units and no split, 3584 x 18944 with 8 ranges, 896 units).  A
// function of the shape only.
#ifndef FP4Q_DEC_UNITS
#define FP4Q_DEC_UNITS 896
#endif
constexpr int64_t kDecUnits = FP4Q_DEC_UNITS;
constexpr int64_t kDecMaxSplits = 16;

bool decode_shape(int64_t M, int64_t K) { return M <= kDecMaxM && K % 128 == 0; }

int decode_splits(int64_t M, int64_t N, int64_t K) {
    const int64_t S = (K + BK - 1) / BK, F = frags_of(N);
    if (2 * F >= kDecUnits) return 1;
    int64_t sp = (kDecUnits + F - 1) / F;
    if (sp > S / 2) sp = S / 2;
    if (sp > kDecMaxSplits) sp = kDecMaxSplits;
    while (sp > 1 && sp * M * N * 4 > kMaxPartialBytes) --sp;
    if (sp < 2) return 1;
    const int64_t per = (S + sp - 1) / sp;
    return (int)((S + per - 1) / per);
}

// Partial products in the workspace, after the packed scales: the larger of
// the two kernels' needs, so that the size depends on the shape only.
int workspace_splits(int64_t M, int64_t N, int64_t K) {
    const int tile = splits_for(M, N, K);
    const int dec = decode_shape(M, K) ? decode_splits(M, N, K) : 1;
    const int sp = tile > dec ? tile : dec;
    return sp > 1 ? sp : 0;
}

template <int AR>
void launch_decode_nv_ar(const NvDecParams& p, hipStream_t stream) {
    constexpr int W = dec_waves(AR);
    const int64_t groups = (p.units + W - 1) / W;
    FP4Q_LAUNCH((k_gemm_decode_nv<AR, W>), dim3((unsigned)groups), dim3(W * kWave), 0, stream, p);
}

template <int AR>
void launch_decode_ar(const DecParams& p, hipStream_t stream) {
    constexpr int W = dec_waves(AR);
    const int64_t groups = (p.units + W - 1) / W;
    FP4Q_LAUNCH((k_gemm_decode<AR, W>), dim3((unsigned)groups), dim3(W * kWave), 0, stream, p);
}

}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const int64_t packed = (packed_bytes(M, N, K) + 255) / 256 * 256;
    return (size_t)(packed + (int64_t)workspace_splits(M, N, K) * M * N * 4);
}

int launch_gemm_nvfp4(const GemmNvJob& j, char* msg, size_t msg_len) {
    if (j.M == 0 || j.N == 0) return 0;
    const hipStream_t stream = static_cast<hipStream_t>(j.stream);
    if (j.M <= kDecMaxM) {
        const int sp = decode_splits(j.M, j.N, j.K);
        const int64_t units = frags_of(j.N) * sp;
        if (units > INT32_MAX) {
            snprintf(msg, msg_len, "gemm: %lld x %lld x %lld needs more workgroups than one launch holds",
                     (long long)j.M, (long long)j.N, (long long)j.K);
            return (int)hipErrorInvalidConfiguration;
        }
        float* partial = reinterpret_cast<float*>(j.ws);
        const NvDecParams p{j.a_codes, j.a_scales, j.b_codes, j.b_scales, j.ga, j.gb, j.M, j.N, j.K,
                            (int)((j.K + BK - 1) / BK), sp, units, j.c, j.ct, partial};
        switch ((j.M + 7) / 8) {
            case 1: launch_decode_nv_ar<1>(p, stream); break;
            case 2: launch_decode_nv_ar<2>(p, stream); break;
            case 3: launch_decode_nv_ar<3>(p, stream); break;
            default: launch_decode_nv_ar<4>(p, stream); break;
        }
        if (sp > 1) {
            const int64_t count = j.M * j.N;
            const int64_t rg = std::min<int64_t>((count + 1023) / 1024, 8192);
            FP4Q_LAUNCH(k_splitk_reduce, dim3((unsigned)rg), dim3(256), 0, stream, partial, sp, count,
                               j.c, j.ct);
        }
        const hipError_t e = hipGetLastError();
        if (e == hipSuccess) return 0;
        snprintf(msg, msg_len, "gemm nvfp4 decode kernel launch: %s", hipGetErrorString(e));
        return (int)e;
    }
    const int64_t tiles = ((j.M + BM - 1) / BM) * ((j.N + BN - 1) / BN);
    const int sp = splits_for(j.M, j.N, j.K);
    if (tiles * sp > INT32_MAX) {
        snprintf(msg, msg_len, "gemm: %lld x %lld x %lld needs more workgroups than one launch holds",
                 (long long)j.M, (long long)j.N, (long long)j.K);
        return (int)hipErrorInvalidConfiguration;
    }
    float* partial = reinterpret_cast<float*>(j.ws);
    const NvParams p{j.a_codes, j.a_scales, j.b_codes, j.b_scales, j.ga, j.gb, j.M, j.N, j.K,
                     j.c, j.ct, sp, partial};
    FP4Q_LAUNCH(k_gemm_nvfp4, dim3((unsigned)(tiles * sp)), dim3(kThreads), 0, stream, p);
    if (sp > 1) {
        const int64_t count = j.M * j.N;
        const int64_t groups = std::min<int64_t>((count + 1023) / 1024, 8192);
        FP4Q_LAUNCH(k_splitk_reduce, dim3((unsigned)groups), dim3(256), 0, stream, partial, sp, count,
                           j.c, j.ct);
    }
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess) return 0;
    snprintf(msg, msg_len, "gemm nvfp4 kernel launch: %s", hipGetErrorString(e));
    return (int)e;
}

size_t gemm_nvfp4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const int sp = M <= kDecMaxM ? decode_splits(M, N, K) : splits_for(M, N, K);
    return sp > 1 ? (size_t)sp * (size_t)M * (size_t)N * 4 : 0;
}

int launch_gemm(const GemmJob& j, char* msg, size_t msg_len) {
    if (j.M == 0 || j.N == 0) return 0;
    const hipStream_t stream = static_cast<hipStream_t>(j.stream);
    const int64_t S = (j.K + BK - 1) / BK;
    float* partial_area = reinterpret_cast<float*>(static_cast<uint8_t*>(j.ws) +
                                                   (packed_bytes(j.M, j.N, j.K) + 255) / 256 * 256);
    if (decode_shape(j.M, j.K) && reinterpret_cast<uintptr_t>(j.a_scales) % 4 == 0 &&
        reinterpret_cast<uintptr_t>(j.b_scales) % 4 == 0) {
        const int sp = decode_splits(j.M, j.N, j.K);
        const int64_t units = frags_of(j.N) * sp;
        if (units > INT32_MAX) {
            snprintf(msg, msg_len, "gemm: %lld x %lld x %lld needs more workgroups than one launch holds",
                     (long long)j.M, (long long)j.N, (long long)j.K);
            return (int)hipErrorInvalidConfiguration;
        }
        const DecParams p{j.a_codes, j.a_scales, j.b_codes, j.b_scales, j.M, j.N, j.K, (int)S, sp, units,
                          j.c, j.ct, partial_area};
        switch ((j.M + 7) / 8) {
            case 1: launch_decode_ar<1>(p, stream); break;
            case 2: launch_decode_ar<2>(p, stream); break;
            case 3: launch_decode_ar<3>(p, stream); break;
            default: launch_decode_ar<4>(p, stream); break;
        }
        if (sp > 1) {
            const int64_t count = j.M * j.N;
            const int64_t rg = std::min<int64_t>((count + 1023) / 1024, 8192);
            FP4Q_LAUNCH(k_splitk_reduce, dim3((unsigned)rg), dim3(256), 0, stream, partial_area, sp,
                               count, j.c, j.ct);
        }
        const hipError_t e = hipGetLastError();
        if (e == hipSuccess) return 0;
        snprintf(msg, msg_len, "gemm decode kernel launch: %s", hipGetErrorString(e));
        return (int)e;
    }
    uint8_t* a_pack = static_cast<uint8_t*>(j.ws);
    uint8_t* b_pack = a_pack + frags_of(j.M) * S * kPackBytes;
    const int64_t kb = j.K / 32;
    const int64_t tiles = ((j.M + BM - 1) / BM) * ((j.N + BN - 1) / BN);
    if (tiles > INT32_MAX || (frags_of(j.M) + frags_of(j.N)) * ((S + kPackStages - 1) / kPackStages) > INT32_MAX) {
        snprintf(msg, msg_len, "gemm: %lld x %lld x %lld needs more workgroups than one launch holds",
                 (long long)j.M, (long long)j.N, (long long)j.K);
        return (int)hipErrorInvalidConfiguration;
    }
    const int64_t runs = (S + kPackStages - 1) / kPackStages;
    const PackOperand pa{j.a_scales, j.M, frags_of(j.M) * runs, reinterpret_cast<uint32_t*>(a_pack)};
    const PackOperand pb{j.b_scales, j.N, frags_of(j.N) * runs, reinterpret_cast<uint32_t*>(b_pack)};
    if (pa.groups + pb.groups > 0)  // none when K = 0
        FP4Q_LAUNCH(k_pack_scales, dim3((unsigned)(pa.groups + pb.groups)), dim3(kPackThreads), 0,
                           stream, pa, pb, kb, S);
    const int sp = splits_for(j.M, j.N, j.K);
    float* partial = partial_area;
    GParams p{j.a_codes, j.b_codes, a_pack, b_pack, j.M, j.N, j.K, S, j.c, j.ct, sp, partial};
    FP4Q_LAUNCH(k_gemm_mxfp4, dim3((unsigned)(tiles * sp)), dim3(kThreads), 0, stream, p);
    if (sp > 1) {
        const int64_t count = j.M * j.N;
        const int64_t groups = std::min<int64_t>((count + 1023) / 1024, 8192);
        FP4Q_LAUNCH(k_splitk_reduce, dim3((unsigned)groups), dim3(256), 0, stream, partial, sp,
                           count, j.c, j.ct);
    }
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess) return 0;
    snprintf(msg, msg_len, "gemm kernel launch: %s", hipGetErrorString(e));
    return (int)e;
}

}  // namespace fp4q
