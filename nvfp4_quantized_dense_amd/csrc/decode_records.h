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
#include "device_common.h"
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

// The down projection's last K split adds the partial sums that the other
// ksplit - 1 splits left as records for output rows 16 r.. (part + (sp * RG
// + r) * 16 + row), in split order, for the lanes that hold token 0 (rows
// 4 q .. 4 q + 3 at lane 16 q). Lane 16 q + sp waits for split sp's four
// records, so all splits are waited for at once (one round trip in all when
// they are already written), and the sums go through the lanes in split
// order. A wait that runs out gives NaN for what was missing and sets the
// status flag.
__device__ __forceinline__ f32x4 sum_split_partials(const uint64_t* part, int64_t RG, int64_t r, int ksplit,
                                                   uint32_t tag, int spin_limit, uint32_t* status, int lane) {
  const int q = lane >> 4, sp = lane & 15;
  const uint64_t* p = part + (sp * RG + r) * 16 + 4 * q;
  uint64_t v[4] = {0, 0, 0, 0};
  uint32_t pending = sp + 1 < ksplit ? 0xFu : 0u;
  for (int spin = 0;; ++spin) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (pending & (1u << k)) v[k] = get_record(p + k);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if ((pending & (1u << k)) && (uint32_t)(v[k] >> 32) == tag) pending &= ~(1u << k);
    if (__all(pending == 0)) break;
    if (spin >= spin_limit) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (pending & (1u << k)) v[k] = __float_as_uint(__builtin_nanf(""));
      if (lane == 0) report_expired(status);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s + 1 < ksplit; ++s) {
#pragma unroll
    for (int k = 0; k < 4; ++k) sum[k] += __uint_as_float((uint32_t)__shfl((int)(uint32_t)v[k], 16 * q + s));
  }
  return sum;
}
#endif

}  // namespace nvfp4
