// The few HIP runtime entry points the host side of the C ABI calls, as host-only stand-ins (C linkage,
// the runtime's status values: 0 success), so that the sanitizer build runs without a GPU or the HIP
// runtime: the RoPE table copy, event records, the current device and its compute-unit count (256, an
// MI355X), the static scratch's address, and the registration calls the compiler emits for the
// file-scope device array.
#include <cstddef>
#include <cstdint>
#include <cstring>

namespace {
alignas(256) unsigned char g_scratch_stand_in[32u << 20];
}

extern "C" {
int hipMemcpyAsync(void* dst, const void* src, size_t bytes, int kind, void* stream) {
  (void)stream;
  // the one copy the ABI makes is host -> device (the RoPE table); the stand-in "device" memory is host
  // memory here, so the copy is real and the sanitizer checks both ranges
  if (kind == 1) std::memcpy(dst, src, bytes);
  return 0;
}
int hipEventRecord(void* event, void* stream) {
  (void)stream;
  return event ? 0 : 400;
}
int hipGetDevice(int* dev) {
  *dev = 0;
  return 0;
}
int hipDeviceGetAttribute(int* value, int attr, int dev) {
  (void)attr, (void)dev;
  *value = 256;
  return 0;
}
int hipGetSymbolAddress(void** ptr, const void* symbol) {
  (void)symbol;
  *ptr = g_scratch_stand_in;
  return 0;
}
void** __hipRegisterFatBinary(const void* data) {
  (void)data;
  static void* handle = nullptr;
  return &handle;
}
void __hipUnregisterFatBinary(void** handle) { (void)handle; }
void __hipRegisterVar(void** handle, char* host_var, char* device_address, const char* device_name, int ext,
                      size_t size, int constant, int global) {
  (void)handle, (void)host_var, (void)device_address, (void)device_name, (void)ext, (void)size, (void)constant,
      (void)global;
}
void __hipRegisterFunction(void** handle, const void* host_fn, char* device_fn, const char* device_name,
                           unsigned int thread_limit, void* tid, void* bid, void* block_dim, void* grid_dim,
                           int* wg_size) {
  (void)handle, (void)host_fn, (void)device_fn, (void)device_name, (void)thread_limit, (void)tid, (void)bid,
      (void)block_dim, (void)grid_dim, (void)wg_size;
}
}
