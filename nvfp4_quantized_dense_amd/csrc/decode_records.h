// decode_records.h -- the tagged records through which the workgroups of a
// single-launch decode MLP (decode.hip, decode16.hip) hand each other h and
// the down projection's partial sums.
//
// A record is one 64-bit word written by one atomic store: 32 bits of data
// and a 32-bit tag, the low half of the launch's epoch (never 0, so a
// zero-filled workspace holds no valid record). Reading the word with a
// device-scope atomic load gives the data and the proof that it belongs to
// this launch in one access: a producer never waits for its stores, and a
// consumer needs no separate flag. Every launch has a new epoch, so a record
// left by an earlier launch is never taken for a current one.
#pragma once
#include "kernels.h"

namespace nvfp4 {

#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ void put_record(uint64_t* p, uint32_t data, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | data, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get_record(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A bounded wait that gave up: the workspace's status word learns of it.
__device__ __forceinline__ void report_expired(uint32_t* status) {
  __hip_atomic_fetch_or(status, kDecodeWaitExpired, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
#endif

}  // namespace nvfp4
