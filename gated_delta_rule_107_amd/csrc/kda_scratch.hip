// The segment workspace of kda_chunk_fwd_noalloc: device memory owned by the library, for
// callers that cannot allocate.  Every GPU the library runs on holds its own copy of the array
// until the process ends.  Host code never passes the array's name to a kernel (on the host it
// names a stand-in, not device memory): it uses the per-device address looked up here.
#include <mutex>
#include <vector>

#include "kda.h"
#include "kda_internal.h"

namespace kda {

static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

hipError_t scratch_address(void** out) {
    static std::mutex mu;
    static std::vector<void*> addr;            // per device, looked up once with it current
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(mu);
    if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

}  // namespace kda
