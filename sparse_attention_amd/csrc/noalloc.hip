// noalloc.hip -- dsa_decode_step_noalloc: the fused step over a scratch array
// the library holds, for callers that cannot allocate (code under graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The scratch array is a file-scope device array of DSA_NOALLOC_SCRATCH_BYTES
// bytes; each device the library runs on holds its own copy until the process
// ends.  In host code the array's name is only a stand-in, so its device
// address is looked up with hipGetSymbolAddress once per device (with that
// device current, on the entry point's first call there) and only that
// address is handed to kernels.  Nothing in the step needs the scratch
// cleared: every region it reads (score rows, row lists, top-k state, split
// partials) is written earlier in the same call.  All calls on one device
// share its array, so calls that overlap on one device race.
#include <mutex>

#include "dsa.h"
#include "dsa_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[DSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device

// The current device's scratch address (nullptr on failure).
void* current_scratch()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" dsa_status_t dsa_decode_step_noalloc(const dsa_rows_t* rows, const void* q_idx, const float* w,
                                                const void* k_idx, float index_scale, const void* q_abs,
                                                const void* kv_latent, float softmax_scale, int32_t k,
                                                int32_t* indices, float* out_latent, float* out_lse,
                                                void* hip_stream)
{
    return dsa::decode_step_in_scratch(rows, q_idx, w, k_idx, index_scale, q_abs, kv_latent, softmax_scale, k,
                                       indices, out_latent, out_lse, DSA_NOALLOC_SCRATCH_BYTES, current_scratch,
                                       hip_stream);
}
