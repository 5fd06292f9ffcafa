// HIP runtime stand-ins for the host-only sanitizer build of the library
// (test infrastructure; never part of libattn.so).
//
// The library's sources are compiled host-only (no device code) under
// AddressSanitizer and UndefinedBehaviorSanitizer and linked against these
// stubs instead of the HIP runtime, so the argument checks, path selection,
// split planning and host merge of the C ABI run on any machine, with no GPU
// and no kernel ever launched.  Every runtime call that would touch a device
// fails with hipErrorNoDevice, so a call that passes validation returns
// ATTN_E_HIP; module registration is a no-op.
#include <stddef.h>
#include <stdint.h>

namespace {
constexpr int kNoDevice = 100;  // hipErrorNoDevice
struct Dim3 {
  uint32_t x, y, z;
};
void* g_handle[1];
}  // namespace

extern "C" {

void** __hipRegisterFatBinary(const void*) { return g_handle; }
void __hipUnregisterFatBinary(void**) {}
void __hipRegisterFunction(void**, const void*, char*, const char*, unsigned int, void*, void*,
                           void*, void*, int*) {}
void __hipRegisterVar(void**, void*, char*, char*, int, size_t, int, int) {}

int __hipPushCallConfiguration(Dim3, Dim3, size_t, void*) { return 0; }
int __hipPopCallConfiguration(Dim3* grid, Dim3* block, size_t* shmem, void** stream) {
  *grid = Dim3{1, 1, 1};
  *block = Dim3{1, 1, 1};
  *shmem = 0;
  *stream = nullptr;
  return 0;
}
int hipLaunchKernel(const void*, Dim3, Dim3, void**, size_t, void*) { return kNoDevice; }
int hipGetLastError(void) { return kNoDevice; }
const char* hipGetErrorString(int) { return "no device (host-only sanitizer build)"; }

int hipGetDevice(int* dev) {
  *dev = 0;
  return kNoDevice;
}
int hipMallocAsync(void** p, size_t, void*) {
  *p = nullptr;
  return kNoDevice;
}
int hipFreeAsync(void*, void*) { return kNoDevice; }
int hipStreamIsCapturing(void*, int* status) {
  *status = 0;  // hipStreamCaptureStatusNone
  return kNoDevice;
}
int hipDeviceGetDefaultMemPool(void** pool, int) {
  *pool = nullptr;
  return kNoDevice;
}
int hipMemPoolSetAttribute(void*, int, void*) { return kNoDevice; }
int hipGetSymbolAddress(void** p, const void*) {
  *p = nullptr;
  return kNoDevice;
}

}  // extern "C"
