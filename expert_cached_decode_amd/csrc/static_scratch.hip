// The library's static device scratch: the step buffers and activations of moe_decode_layer_static,
// for callers that cannot allocate device memory. One file-scope device array per GPU (each device
// that loads the library holds its own copy until the process ends); host code reaches it only
// through the device address hipGetSymbolAddress returns for the current device, kept per device.
#include <mutex>

#include "ec_internal.h"

namespace ec {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];         // device address of `scratch` on each device (null until set up)
bool g_cleared[kMaxDevices];      // the device's copy has been zeroed once
} // namespace

// Device address of the scratch array on the current device, looked up once per device (the
// current device must be `device`). Null with *err set on failure.
void* static_scratch_ptr(int device, hipError_t* err) {
    *err = hipSuccess;
    if (device < 0 || device >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[device]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
            return nullptr;
        }
        g_ptr[device] = p;
    }
    return g_ptr[device];
}

// Zero the device's scratch once (a fill kernel on `s`, so the clearing can sit in a captured graph),
// before its first use.
void static_scratch_clear_once(int device, void* ptr, hipStream_t s) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (device < 0 || device >= kMaxDevices || g_cleared[device]) return;
    launch_fill_i32(reinterpret_cast<int32_t*>(ptr), 0, (int64_t)(kStaticScratchBytes / 4), s);
    g_cleared[device] = true;
}

} // namespace ec
