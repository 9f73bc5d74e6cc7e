// Next unit of a workgroup under the queue schedule of kda_verify.hip, kept in its own
// header so that a host-only test can compile and check it on the CPU.
//
// The queue launches `resident` workgroups over `units` units (resident <= units). Units
// [0, resident) are the first round, one per workgroup by its index. After that, ticket k
// (the value a workgroup drew from the workspace counter, which starts at 0 and counts up
// by one per draw) names unit resident + k. The result is that unit, or -1 once the
// tickets have passed the last unit. The test is an unsigned comparison over the whole
// 32-bit ticket, so a counter holding any value at all (a call that did not run to
// completion leaves it non-zero) ends the loop at once rather than forming a negative or
// out-of-range unit; the sum resident + k is then below units, so it cannot overflow.
#ifndef KDA_QUEUE_H
#define KDA_QUEUE_H

#include <stdint.h>

#ifndef KDA_HOST_DEVICE
#define KDA_HOST_DEVICE
#endif

static inline KDA_HOST_DEVICE int kda_queue_unit(uint32_t ticket, int units, int resident) {
  const uint32_t rest = units > resident ? (uint32_t)(units - resident) : 0u;
  return ticket < rest ? resident + (int)ticket : -1;
}

#endif  // KDA_QUEUE_H
