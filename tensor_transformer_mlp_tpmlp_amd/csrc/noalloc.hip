// The forward pass for callers that cannot allocate device memory (code
// under stream capture, tight serving loops, harnesses that forbid
// hipMalloc): tpmlp_forward_noalloc runs tpmlp_forward_ex with its
// workspace taken from a fixed array in the library's own device memory.
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on
// holds its own copy, allocated with the code object and kept until the
// process ends.  In host code the name `scratch` is only the host-side
// shadow of that array, never a device address, so the device address is
// looked up once per device (hipGetSymbolAddress with that device current)
// and that pointer, not the name, is what the kernels receive.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/tpmlp.h"

static_assert(TPMLP_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte blocks");

// Nothing in it needs to start at zero: the forward writes every byte of
// its workspace that it later reads (H, the LayerNorm statistics, the fp32
// sum of the Norm-after placement).  It keeps the last call's contents.
static __device__ __align__(256) unsigned char scratch[TPMLP_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = TPMLP_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

struct DeviceScratch {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
DeviceScratch g_dev[kMaxDevices];

// The current device's copy of `scratch` (looked up on the first call on
// that device); nullptr if the device index is out of range or the lookup
// failed.
void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    DeviceScratch& d = g_dev[dev];
    std::call_once(d.once, [&d] {
        void* p = nullptr;
        d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        d.ptr = d.err == hipSuccess ? p : nullptr;
    });
    return d.ptr;
}

}  // namespace

extern "C" tpmlp_status tpmlp_forward_noalloc(const void* X, int64_t M, const tpmlp_shards* s, void* Y,
                                              const tpmlp_opts* opts, void* stream) {
    if (!s) return TPMLP_ERR_NULL;
    if (M < 0) return TPMLP_ERR_SHAPE;
    tpmlp_opts o;
    tpmlp_opts_init(&o);
    if (opts) o = *opts;
    if (o.workspace) return TPMLP_ERR_WORKSPACE;  // the scratch array is the workspace
    if (M == 0) return tpmlp_forward_ex(X, M, s, Y, &o, stream);
    const size_t need = tpmlp_forward_workspace_bytes(s, M, o.flags, o.shard_index >= 0 ? 1 : 0);
    if (need == 0) return TPMLP_ERR_SHAPE;       // invalid sizes or flags
    if (need > kScratchBytes) return TPMLP_ERR_WORKSPACE;
    void* ws = scratch_for_current_device();
    if (!ws) return TPMLP_ERR_HIP;
    o.workspace = ws;
    o.workspace_bytes = kScratchBytes;
    return tpmlp_forward_ex(X, M, s, Y, &o, stream);
}
