// The device-side precondition word read by sv_check_device_errors.
//
// A build with SV_DEBUG keeps one 32-bit word per GPU in this file's device
// memory; the kernels OR a bit into it when they meet a broken device-side
// input (see SV_DEVERR_* in sv.h).  Host code reaches the word through its
// device address, looked up once per device with hipGetSymbolAddress (in host
// code the symbol's own name is only a stand-in, not a device address).
#include "device_common.h"

namespace sv {

#ifdef SV_DEBUG
namespace {

__device__ __attribute__((aligned(256))) unsigned int dev_error_word[1] = {};

constexpr int kMaxDevices = 64;
// per device: the word's address, looked up on the first use (two threads
// that race here store the same value)
unsigned int *g_word[kMaxDevices] = {};
bool g_word_done[kMaxDevices] = {};

}  // namespace

unsigned int *device_error_word() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    if (!__atomic_load_n(&g_word_done[dev], __ATOMIC_ACQUIRE)) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(dev_error_word)) != hipSuccess) return nullptr;
        g_word[dev] = (unsigned int *)ptr;
        __atomic_store_n(&g_word_done[dev], true, __ATOMIC_RELEASE);
    }
    return g_word[dev];
}
#else
unsigned int *device_error_word() { return nullptr; }
#endif

}  // namespace sv

extern "C" int sv_check_device_errors(void *stream) {
#ifdef SV_DEBUG
    unsigned int *word = sv::device_error_word();
    if (word == nullptr) return sv::hip_fail(hipErrorInvalidDevice);
    hipStream_t st = (hipStream_t)stream;
    unsigned int bits = 0;
    const unsigned int zero = 0;
    hipError_t e = hipMemcpyAsync(&bits, word, sizeof(bits), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipMemcpyAsync(word, &zero, sizeof(zero), hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return sv::hip_fail(e);
    return (int)(bits & 0x7fffffffu);
#else
    (void)stream;
    return 0;
#endif
}
