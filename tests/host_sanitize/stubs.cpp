// Host-only stand-ins for the HIP runtime calls and kernel launches that the C-ABI layer
// (relative_bias_gqa_amd/csrc/abi.cpp) makes, so that the layer can be built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer and driven on a machine without a GPU.
// Each launch records its parameters for the driver to check; no kernel runs.
#include <hip/hip_runtime.h>

#include <cstring>

#include "backward.hpp"
#include "launch.hpp"
#include "stubs.hpp"

namespace stub {
Record rec;
}

extern "C" hipError_t hipGetDevice(int* device) {
  *device = stub::rec.device;
  return hipSuccess;
}

extern "C" hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int device) {
  (void)device;
  *value = attr == hipDeviceAttributeMultiprocessorCount ? stub::rec.compute_units : 0;
  return hipSuccess;
}

extern "C" const char* hipGetErrorString(hipError_t) { return "host stub"; }

namespace rattn {

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t) {
  stub::rec.prefill = p;
  ++stub::rec.prefill_bf16_calls;
  return hipSuccess;
}

hipError_t launch_prefill_fp32(const PrefillParams& p, hipStream_t) {
  stub::rec.prefill = p;
  ++stub::rec.prefill_fp32_calls;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t) {
  stub::rec.decode = p;
  ++stub::rec.decode_calls;
  if (!stub::rec.on_decode(p)) return hipErrorInvalidValue;
  return hipSuccess;
}

hipError_t launch_sconv_write(const SconvParams& p, hipStream_t) {
  stub::rec.sconv = p;
  ++stub::rec.sconv_calls;
  return hipSuccess;
}

hipError_t launch_backward(const BackwardParams& p, hipStream_t) {
  stub::rec.backward = p;
  ++stub::rec.backward_calls;
  return hipSuccess;
}

// the allocation-free decode's static scratch: a host array of the same size
static unsigned char host_scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  *ptr = host_scratch;
  return hipSuccess;
}

}  // namespace rattn

namespace stub {
const void* scratch_base() { return rattn::host_scratch; }
}  // namespace stub
