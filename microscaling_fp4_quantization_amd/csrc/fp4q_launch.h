// Internal interface between the C ABI layer (fp4q_abi.cpp) and the kernel
// launchers (fp4q_kernels.hip).  Plain types only; arguments arrive here
// already validated.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace fp4q {

// Workspace layout (bytes from the start of ws).  Every slot is written before
// it is read within one call, so the workspace needs no initial contents.
constexpr int kMaxGroups = 16384;           // upper bound on any grid size
constexpr size_t kWsAmax = 0;               // uint32 per-workgroup |x| maxima
// Per-workgroup error terms, one array per term (structure of arrays):
// [non-max | max | zero-rounding | sum x^2] as double, then the zero-block count.
constexpr size_t kWsPartials = kWsAmax + 4 * (size_t)kMaxGroups;
// sum x^2 per workgroup of the amax pre-pass (dynamic mode), as double
constexpr size_t kWsAmaxSumsq = kWsPartials + 5 * 8 * (size_t)kMaxGroups;
constexpr size_t kWsBytes = kWsAmaxSumsq + 8 * (size_t)kMaxGroups;

struct QuantJob {
    const void* x;
    int xt;            // 0 bf16, 1 f32
    int64_t n;         // rows * cols
    int64_t rows, cols;
    int block;         // 8..256
    int fmt;           // 0 MXFP4, 1 UE4M3, 2 UE5M3
    int gmode;         // 0 none, 1 dynamic, 2 given, 3 per row
    float* g;          // device: dynamic out / given in / one per row out
    int rotate;        // 0, 16, 32
    uint8_t* codes;
    uint8_t* scales;
    float* block_mse;  // nullable
    int mse_kind;      // 0 abs, 1 rel
    void* stats;       // nullable, fp4q_stats layout
    void* ws;
    void* stream;
    int radius = -1;   // >= 0: per-block scale search over this many neighbours
    // MXFP4 pass of fp4_quantize_mx_nv: the quantize kernel also writes its
    // per-workgroup max |x| (binary32 bits) to amax_out, and the reduction
    // kernel turns them into the NVFP4 per-tensor scale at g_from_amax.
    uint32_t* amax_out = nullptr;
    float* g_from_amax = nullptr;
    // NVFP4 pass of fp4_quantize_mx_nv: stores with the nontemporal bit.
    bool nv_of_pair = false;
};

struct DequantJob {
    const uint8_t* codes;
    const uint8_t* scales;
    int fmt;
    int block;
    const float* g;    // nullable (UE4M3)
    int64_t n;
    int rotate;
    void* out;
    int ot;            // 0 bf16, 1 f32
    void* stream;
};

struct MseJob {
    const void* x;
    int xt;
    const uint8_t* codes;
    const uint8_t* scales;
    int fmt;
    int block;
    const float* g;    // nullable (UE4M3)
    int64_t n;
    int rotate;
    float* block_mse;
    int mse_kind;
    void* stats;
    void* ws;
    void* stream;
};

struct RotateJob {
    const void* x;
    int xt;
    int64_t n;
    int rotate;
    float* out;
    void* stream;
};

struct GemmJob {
    const uint8_t* a_codes;
    const uint8_t* a_scales;
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    int64_t M, N, K;
    void* c;
    int ct;            // 0 bf16, 1 f32
    void* ws;          // gemm_workspace_bytes(M, N, K) bytes: packed scales
    void* stream;
};

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

struct GemmNvJob {
    const uint8_t* a_codes;
    const uint8_t* a_scales;  // UE4M3 per 16 elements
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    const float* ga;          // per-tensor scales (device), nullable
    const float* gb;
    int64_t M, N, K;
    void* c;
    int ct;                   // 0 bf16, 1 f32
    void* ws;                 // gemm_nvfp4_workspace_bytes(M, N, K) bytes: partials
    void* stream;
};

size_t gemm_nvfp4_workspace_bytes(int64_t M, int64_t N, int64_t K);

// Launch timing (fp4q_profile_events): while the calling thread has event
// pairs left, every kernel launch records the next pair on its stream around
// itself.  Streams and events are passed as void*.
void profile_set(void* const* events, int n_pairs);
int profile_count();
void profile_before(void* stream);
void profile_after(void* stream);

// A kernel launch bracketed by the timing hooks (used for every launch).
#define FP4Q_LAUNCH(kernel, grid, block, shmem, stream, ...)                       \
    do {                                                                           \
        ::fp4q::profile_before(stream);                                            \
        hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);       \
        ::fp4q::profile_after(stream);                                             \
    } while (0)

// The library's static device scratch for the allocation-free entry point:
// its device address on the current device (looked up once per device) and
// its size (kWsBytes).  Returns 0, else a HIP error code with `msg` set.
int scratch_workspace(void** ptr, size_t* bytes, char* msg, size_t msg_len);

// Each returns 0 on success, else a HIP error code; `msg` gets a description.
int launch_quantize(const QuantJob& j, char* msg, size_t msg_len);
// MXFP4 (mx) then dynamic NVFP4 (nv) of the same unrotated tensor, the NVFP4
// per-tensor scale taken from the MXFP4 pass's maxima (no amax pass).
int launch_quantize_mx_nv(const QuantJob& mx, const QuantJob& nv, char* msg, size_t msg_len);
// The same for n <= kMaxBatchTensors tensors in one launch per pass: mx[i] and
// nv[i] describe tensor i (same dtype, NVFP4 block 16 or 32, and the same
// outputs wanted for every tensor); one reduction launch per pass.
constexpr int kMaxBatchTensors = 16;
int launch_quantize_mx_nv_batch(const QuantJob* mx, const QuantJob* nv, int n, char* msg,
                                size_t msg_len);
int launch_dequantize(const DequantJob& j, char* msg, size_t msg_len);
int launch_block_mse(const MseJob& j, char* msg, size_t msg_len);
int launch_rotate(const RotateJob& j, char* msg, size_t msg_len);
int launch_gemm(const GemmJob& j, char* msg, size_t msg_len);
int launch_gemm_nvfp4(const GemmNvJob& j, char* msg, size_t msg_len);

}  // namespace fp4q
