// Launch records of the host stubs (tests/host_sanitize/stubs.cpp).
#pragma once

#include <functional>

#include "backward.hpp"
#include "launch.hpp"

namespace stub {

struct Record {
  int compute_units = 256;
  // the current device's index: the library caches the compute-unit count per device, so each
  // count the driver tries is reported for a device of its own
  int device = 0;
  rattn::PrefillParams prefill{};
  rattn::DecodeParams decode{};
  rattn::SconvParams sconv{};
  rattn::BackwardParams backward{};
  int prefill_bf16_calls = 0, prefill_fp32_calls = 0, decode_calls = 0, sconv_calls = 0, backward_calls = 0;
  // called on every decode launch (a call may launch several batches); false fails the launch
  std::function<bool(const rattn::DecodeParams&)> on_decode = [](const rattn::DecodeParams&) { return true; };
};

extern Record rec;
const void* scratch_base();

}  // namespace stub
