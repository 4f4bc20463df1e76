// fp4q_scratch.hip -- the fixed device scratch of the allocation-free entry
// point (nvfp4_quantize_noalloc).
//
// The array holds one call's workgroup partials and amax maxima: kWsBytes, a
// constant, since grids never exceed kMaxGroups workgroups and so any tensor
// size fits.  Each device holds its own copy for the life of the process.  On
// the host the array's name is only a stand-in for it; its device address
// comes from hipGetSymbolAddress, looked up once per device with that device
// current, and kept.  The contents need no initial value: every slot is
// written before it is read within one call.  All such calls on one device
// share the array, so calls that overlap on one device race.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdio.h>

#include <mutex>

#include "fp4q_launch.h"

namespace fp4q {

static __device__ __align__(256) uint8_t scratch[kWsBytes];

namespace {
constexpr int kMaxDevices = 64;
}  // namespace

int scratch_workspace(void** ptr, size_t* bytes, char* msg, size_t msg_len) {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        snprintf(msg, msg_len, "hipGetDevice: %s", hipGetErrorString(e));
        return (int)e;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        snprintf(msg, msg_len, "device %d is beyond the %d devices the scratch table holds", dev,
                 kMaxDevices);
        return (int)hipErrorInvalidDevice;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) {
            snprintf(msg, msg_len, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
            return (int)e;
        }
        addr[dev] = p;
    }
    *ptr = addr[dev];
    *bytes = sizeof(scratch);
    return 0;
}

}  // namespace fp4q
