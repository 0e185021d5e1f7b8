// How many workgroups of a launch shape a CU really holds at once, for kernels
// that keep different numbers of scalar registers per wave.  The first lane of
// every workgroup records the hardware ids of the CU it runs on (HW_ID with
// its XCC id) and the device's realtime counter before and after a bounded
// sleep; no workgroup waits on another, so every launch ends after about
// grid / resident-per-GPU rounds of the sleep.  The host reads the intervals
// and counts how many overlap on each CU.
//
// The three builds differ only in the scalar registers the compiler has to
// set aside: an empty asm statement that names s10..sTOP as clobbered keeps
// the compiler's own values above sTOP, so the wave holds about TOP + 7 SGPRs
// (level 0: no clobber, about 20; level 1: TOP 81, about 88; level 2: TOP 97,
// about 104).  The split-row planner's residency table depends on how many
// waves such kernels fit on a SIMD, which neither the compiler's occupancy
// report nor the runtime's occupancy query gets right on this part.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "fused_boundary.h"

namespace {

#define FB_S10_19 "s10", "s11", "s12", "s13", "s14", "s15", "s16", "s17", "s18", "s19"
#define FB_S20_29 "s20", "s21", "s22", "s23", "s24", "s25", "s26", "s27", "s28", "s29"
#define FB_S30_39 "s30", "s31", "s32", "s33", "s34", "s35", "s36", "s37", "s38", "s39"
#define FB_S40_49 "s40", "s41", "s42", "s43", "s44", "s45", "s46", "s47", "s48", "s49"
#define FB_S50_59 "s50", "s51", "s52", "s53", "s54", "s55", "s56", "s57", "s58", "s59"
#define FB_S60_69 "s60", "s61", "s62", "s63", "s64", "s65", "s66", "s67", "s68", "s69"
#define FB_S70_79 "s70", "s71", "s72", "s73", "s74", "s75", "s76", "s77", "s78", "s79"
#define FB_S80_81 "s80", "s81"
#define FB_S82_97 "s82", "s83", "s84", "s85", "s86", "s87", "s88", "s89", "s90", "s91", "s92", \
                  "s93", "s94", "s95", "s96", "s97"

template <int LEVEL>
__global__ void __launch_bounds__(1024) residency_probe_kernel(unsigned long long* out,
                                                               unsigned long long ticks) {
  if constexpr (LEVEL >= 1)
    asm volatile("" ::: FB_S10_19, FB_S20_29, FB_S30_39, FB_S40_49, FB_S50_59, FB_S60_69,
                 FB_S70_79, FB_S80_81);
  if constexpr (LEVEL >= 2) asm volatile("" ::: FB_S82_97);
  if (threadIdx.x == 0) {
    const unsigned hw_id = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_ID, 32 bits
    const unsigned xcc_id = __builtin_amdgcn_s_getreg((15 << 11) | 20); // XCC_ID, 16 bits
    const unsigned long long t0 = wall_clock64();
    while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(10);
    const unsigned long long t1 = wall_clock64();
    out[3 * (size_t)blockIdx.x + 0] = ((unsigned long long)xcc_id << 32) | hw_id;
    out[3 * (size_t)blockIdx.x + 1] = t0;
    out[3 * (size_t)blockIdx.x + 2] = t1;
  }
  __syncthreads();  // every wave of the workgroup stays until the sleep ends
}

}  // namespace

extern "C" int fused_boundary_residency_probe(int32_t sgpr_level, int32_t grid, int32_t block,
                                              uint64_t sleep_ticks, void* out, void* stream) {
  if (sgpr_level < 0 || sgpr_level > 2 || grid <= 0 || grid > 65536 || block < 64 ||
      block > 1024 || block % 64 != 0 || sleep_ticks > 1000000ull || out == nullptr ||
      ((uintptr_t)out & 7u))
    return FB_INVALID_ARGUMENT;
  unsigned long long* o = (unsigned long long*)out;
  const unsigned long long t = sleep_ticks;
  void* args[] = {&o, (void*)&t};
  const void* fn = sgpr_level == 0   ? reinterpret_cast<const void*>(residency_probe_kernel<0>)
                   : sgpr_level == 1 ? reinterpret_cast<const void*>(residency_probe_kernel<1>)
                                     : reinterpret_cast<const void*>(residency_probe_kernel<2>);
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3((unsigned)block), args, 0,
                         (hipStream_t)stream) == hipSuccess
             ? FB_OK
             : FB_HIP_ERROR;
}
