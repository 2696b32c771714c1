// static_scratch.hip -- the fixed device buffer behind pa_decode_noalloc: a
// file-scope device array that the library owns for the life of the process,
// so that a call needs no workspace from its caller and allocates nothing.
//
// In host code the array's name is only a host-side stand-in for the symbol,
// not a device address.  Its address on a device comes from
// hipGetSymbolAddress, asked once per device with that device current and
// kept here; every user of the buffer takes that address.
#include <mutex>
#include <vector>

#include "pa_internal.h"

namespace pa {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

int static_scratch(void **ptr)
{
    static std::mutex mu;
    static std::vector<void *> addr;           // per device id
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return PA_ERR_HIP;
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= (int)addr.size())
        addr.resize(dev + 1, nullptr);
    if (!addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return PA_ERR_HIP;
        }
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return PA_OK;
}

}  // namespace pa
