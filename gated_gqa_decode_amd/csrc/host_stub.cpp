// host_stub.cpp -- stand-ins for the HIP runtime calls and kernel launchers
// that capi.cpp makes, so the C ABI's host logic (argument checks, split
// plans, workspace layout, the device-arch decision, the no-allocation
// entry point's scratch lookup) can be linked and exercised on a machine with
// no GPU, and built with host sanitizers.  Linked only into the host-check
// library (build.py, build_host_check); the product library links the real
// runtime and kernels.
//
// Controls (extern "C", for the tests): the architecture name the fake
// device reports, and a record of every launch the ABI would have made.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "ga_internal.h"

namespace {

char g_arch[64] = "gfx950:sramecc+:xnack-";
int g_device_calls = 0;

struct Record {
  int decode = 0, prefill = 0, rope = 0, stream_read = 0;
  ga::DecodeLaunch last_decode{};
  ga::PrefillLaunch last_prefill{};
  ga::RopeLaunch last_rope{};
} g_rec;

const void* g_var_shadow = nullptr;  // host shadow of the registered device variable
constexpr uintptr_t kFakeScratch = 0x7e0000000000ull;

}  // namespace

// ---- the HIP runtime entry points capi.cpp uses ---------------------------
extern "C" {

hipError_t hipGetDevice(int* dev) {
  ++g_device_calls;
  *dev = 0;
  return hipSuccess;
}

hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* prop, int dev) {
  if (dev != 0) return hipErrorInvalidDevice;
  std::memset(prop, 0, sizeof(*prop));
  std::strncpy(prop->gcnArchName, g_arch, sizeof(prop->gcnArchName) - 1);
  return hipSuccess;
}

hipError_t hipGetSymbolAddress(void** ptr, const void* symbol) {
  if (symbol == nullptr || symbol != g_var_shadow) return hipErrorInvalidSymbol;
  *ptr = reinterpret_cast<void*>(kFakeScratch);
  return hipSuccess;
}

// Code-object registration emitted by the compiler for the device variable.
void** __hipRegisterFatBinary(const void*) {
  static void* handle = nullptr;
  return &handle;
}
void __hipUnregisterFatBinary(void**) {}
void __hipRegisterVar(void**, void* var, char*, char*, int, size_t, int, int) {
  g_var_shadow = var;
}

// ---- test controls ----------------------------------------------------------
// The next device-arch query reports `arch` (the ABI caches the answer per
// device, so a test sets it once per process).
void ga_stub_set_arch(const char* arch) {
  std::strncpy(g_arch, arch, sizeof(g_arch) - 1);
  g_arch[sizeof(g_arch) - 1] = 0;
}

// Launches recorded so far: {decode, prefill, qk_norm_rope, stream_read}.
void ga_stub_launch_counts(int* out4) {
  out4[0] = g_rec.decode;
  out4[1] = g_rec.prefill;
  out4[2] = g_rec.rope;
  out4[3] = g_rec.stream_read;
}

// Fields of the last decode launch: tokens_per_split, num_splits,
// split_target, batch, page_size, kv_fp8, window, num_q_heads; and the
// workspace pointers (part_acc, part_ml, out).
void ga_stub_last_decode(int32_t* i8, uint64_t* p3, float* f3) {
  const ga::DecodeLaunch& d = g_rec.last_decode;
  const int32_t v[8] = {d.tokens_per_split, d.num_splits, d.split_target, d.batch,
                        d.page_size,        d.kv_fp8,     d.window,       d.num_q_heads};
  std::memcpy(i8, v, sizeof(v));
  p3[0] = reinterpret_cast<uintptr_t>(d.part_acc);
  p3[1] = reinterpret_cast<uintptr_t>(d.part_ml);
  p3[2] = reinterpret_cast<uintptr_t>(d.out);
  f3[0] = d.scale;
  f3[1] = d.k_descale;
  f3[2] = d.v_descale;
}

int ga_stub_device_calls(void) { return g_device_calls; }

// The launchers' invariant-divisor division, host side (the kernels use the
// same inline function).
uint32_t ga_stub_divu32(uint32_t n, uint32_t d) { return ga::divu32(n, ga::divu32_make(d)); }

}  // extern "C"

// ---- the kernel launchers ------------------------------------------------------
namespace ga {

hipError_t launch_decode(const DecodeLaunch& d, hipStream_t) {
  ++g_rec.decode;
  g_rec.last_decode = d;
  return hipSuccess;
}

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t) {
  ++g_rec.prefill;
  g_rec.last_prefill = p;
  return hipSuccess;
}

hipError_t launch_qk_norm_rope(const RopeLaunch& p, hipStream_t) {
  ++g_rec.rope;
  g_rec.last_rope = p;
  return hipSuccess;
}

hipError_t launch_stream_read(const void*, size_t, uint32_t*, hipStream_t) {
  ++g_rec.stream_read;
  return hipSuccess;
}

}  // namespace ga
