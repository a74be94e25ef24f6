// static_scratch.hip -- the per-device scratch array behind moe_forward_static, for callers
// that cannot allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// The array is a file-scope __device__ object: every GPU the library runs on holds its
// own copy at its own address until the process ends.  On the host its name is only a
// stand-in for the symbol, so host code never passes it to a kernel or a copy; the device
// address is looked up once per device with hipGetSymbolAddress (with that device
// current) and kept, and only that address is used.  Every call on a device shares that
// device's array: calls that overlap on one GPU race.
#include <mutex>

#include "kernels.h"

namespace moe {

static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    bool ready;
    void* ptr;          // device address of this device's copy of `scratch`
    int num_cu;
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

}  // namespace

hipError_t static_scratch(void** ptr, int* num_cu) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceScratch& d = g_dev[dev];
    if (!d.ready) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidSymbol;
        int ncu = 0;
        e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        d.ptr = p;
        d.num_cu = ncu > 0 ? ncu : 256;
        d.ready = true;
    }
    *ptr = d.ptr;
    *num_cu = d.num_cu;
    return hipSuccess;
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

}  // namespace moe
