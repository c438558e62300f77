// kda_noalloc.hip -- kda_prefill_noalloc: the chunkwise prefill for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The prefill's workspace (chunk table, null row, segment records, segment
// transitions and incoming states, and the per-(chunk, head) slabs) lives in
// a file-scope device array of KDA_NOALLOC_SCRATCH_BYTES bytes instead of a
// caller buffer.  Each GPU the library runs on holds its own copy of the
// array, at its own address, until the process ends.  In host code the
// array's name is only a host-side stand-in: its device address is taken
// once per device with hipGetSymbolAddress, with that device current, and
// only that address is ever handed to a kernel.
//
// Every call on a device shares that device's array.  Nothing in it has to
// start at zero: every byte a prefill reads from its workspace is written
// earlier in the same call (the chunk-table kernel writes the table, the
// null row and the segment records; the intra kernel writes every slab the
// inter kernel reads; transitions and incoming states are written before
// the combine and output passes read them).  Calls that overlap in time on
// one device (different streams, or different threads without ordering)
// race on the array and give undefined results.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda.h"

namespace {

static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call on that device; nullptr if the lookup fails.
void *scratch_address() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch[dev] = ptr;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" int kda_prefill_noalloc(kda_dtype io_dtype, const void *q, const void *k, const void *v,
                                   const float *z, const float *A, const float *beta, const float *h0,
                                   const int32_t *cu_seqlens, int N, int T, int H, int dk, int dv, void *o,
                                   float *hT, void *stream) {
    const size_t need = kda_prefill_workspace_size(N, T, H, dk, dv, io_dtype);
    if (need == 0)   // sizes kda_prefill rejects: report its status (no workspace is touched)
        return kda_prefill(io_dtype, q, k, v, z, A, beta, h0, cu_seqlens, N, T, H, dk, dv, o, hT, nullptr, 0,
                           stream);
    if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH_TOO_SMALL;
    void *ws = scratch_address();
    if (!ws) return KDA_ERR_HIP;
    return kda_prefill(io_dtype, q, k, v, z, A, beta, h0, cu_seqlens, N, T, H, dk, dv, o, hT, ws,
                       KDA_NOALLOC_SCRATCH_BYTES, stream);
}
