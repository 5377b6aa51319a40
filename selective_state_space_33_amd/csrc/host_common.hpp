// host_common.hpp -- host-side helpers shared by the C-ABI entry points.
//
// Every workspace starts with kHeaderWords 32-bit words, zeroed by the first
// kernel of each call:
//   word 0  status: the OR of kStatus* bits the call's kernels set (a chained
//           hand-off wait that ran out); read back by ssm_workspace_status;
//   word 1  the workgroup ticket of a chained launch;
//   word 2  the ticket of a second chained launch in the same call;
//   word 3  never written: the word every wait polls instead of its flag when
//           the test hook SSM_TEST_NEVER_READY=1 is set, so that each wait
//           runs out (with SSM_TEST_SPIN_LIMIT polls) and every kernel still
//           ends normally.
// The ready flags of a chained launch follow the header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "common.hpp"

namespace ssm {

constexpr int kHeaderWords = 4;
constexpr int kWordStatus = 0, kWordTicket = 1, kWordTicket2 = 2, kWordNever = 3;

// Compute units of the current device, over which the planners balance the
// work.  SSM_NUM_CU (environment) overrides it, for tests of the planners at
// other sizes; without a device (a size query on a machine with no GPU) the
// MI355X's 256 is assumed.  The count of each device is looked up once.
inline int64_t device_cu_count() {
  const char* e = getenv("SSM_NUM_CU");
  if (e && atoi(e) > 0) return atoi(e);
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return 256;
  }
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  if (dev < 64) cached[dev] = n;
  return n;
}

// Polls per chained wait: kSpinLimit, or SSM_TEST_SPIN_LIMIT (tests).
inline unsigned wait_spin_limit() {
  const char* e = getenv("SSM_TEST_SPIN_LIMIT");
  if (e && atoi(e) > 0) return static_cast<unsigned>(atoi(e));
  return kSpinLimit;
}

// The test hook's never-written word, or null.
inline const unsigned* wait_override(const unsigned* header) {
  const char* e = getenv("SSM_TEST_NEVER_READY");
  return (e && e[0] == '1') ? header + kWordNever : nullptr;
}

}  // namespace ssm
