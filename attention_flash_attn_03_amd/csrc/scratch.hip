// scratch.hip -- the library's static device scratch for callers that cannot
// allocate (attn_paged_decode_noalloc): one array per GPU the library runs on,
// held until the process ends.  Its address on the current device is looked up
// once with hipGetSymbolAddress; host code uses only that address, never the
// array's name (which on the host is a stand-in, not a device address).
#include <mutex>

#include "internal.h"

namespace attn {

static __device__ __align__(256) uint8_t scratch[ATTN_DECODE_SCRATCH_BYTES];

int decode_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex lock;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_EHIP;
    std::lock_guard<std::mutex> guard(lock);
    if (!addr[dev]) {
        void *a = nullptr;
        if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return ATTN_EHIP;
        addr[dev] = a;
    }
    *ptr = addr[dev];
    return ATTN_OK;
}

}  // namespace attn
