// What this part attains for the boundary's own memory traffic: a diagnostic
// kernel with the stream kernel's load pattern and launch shape and none of its
// arithmetic.  Per token row it reads num_direct rows at the row's own offset
// (the partials, shared expert and residual of the boundary) and num_gathered
// rows of one buffer through an index map (the expert gathers), 16-byte
// nontemporal loads, vec_per_thread (1, 2, 4 or 8) vectors per lane, whole rows per
// workgroup, at most workgroups_per_cu resident per CU; then, if asked,
// writes num_outputs rows (the boundary's two outputs) with nontemporal
// stores.  The loaded data is folded with XOR so no load is dead code; the
// written rows are that fold, not a result.  bench.py times it on the
// benchmark's own buffers next to the boundary kernel.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "fused_boundary.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeMaxDirect = FB_MAX_PARTIALS + 2;
constexpr int kProbeMaxOutputs = 2;

struct ProbeArgs {
  const u32x4* direct[kProbeMaxDirect];
  const u32x4* gathered;
  const int32_t* idx;
  u32x4* out[kProbeMaxOutputs];
  int num_direct;
  int num_gathered;
  int num_outputs;
  int H8;
  uint32_t n_rows32;  // rows of the gathered buffer, min(N, 2^31): index e is read iff (uint32)e < this
};

__device__ __forceinline__ int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

template <int VPT>
__global__ void __launch_bounds__(512) probe_kernel(const ProbeArgs a) {
  const int B = blockDim.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int row = blockIdx.x;
  const size_t roff = (size_t)row * (size_t)a.H8;
  // the row's gather indices, one per lane, as the boundary reads its routing
  int my_idx = -1;
  if (lane < a.num_gathered) my_idx = a.idx[(size_t)row * a.num_gathered + lane];
  u32x4 acc[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) acc[j] = u32x4{0u, 0u, 0u, 0u};
  const int nsrc = a.num_direct + a.num_gathered;
  for (int i = 0; i < nsrc; ++i) {
    const u32x4* base;
    if (i < a.num_direct) {
      base = a.direct[i] + roff;
    } else {
      const int e = readlane_i(my_idx, i - a.num_direct);
      if ((uint32_t)e >= a.n_rows32) continue;  // outside the buffer: skipped, as the boundary does
      base = a.gathered + (size_t)e * (size_t)a.H8;
    }
    // branch-free: lanes past the row end read its last vector and drop it, so
    // every load of a source is in flight at once
    u32x4 x[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int v = tid + j * B;
      x[j] = __builtin_nontemporal_load(base + (v < a.H8 ? v : a.H8 - 1));
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j)
      acc[j] ^= tid + j * B < a.H8 ? x[j] : u32x4{0u, 0u, 0u, 0u};
  }
  for (int d = 0; d < a.num_outputs; ++d)
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int v = tid + j * B;
      if (v < a.H8) __builtin_nontemporal_store(acc[j] ^ (uint32_t)d, a.out[d] + roff + v);
    }
}

thread_local int t_probe_hip_error = 0;

}  // namespace

extern "C" int fused_boundary_bandwidth_probe(const void* const* direct, int32_t num_direct,
                                              const void* gathered, int64_t num_gathered_rows,
                                              const int32_t* gather_idx, int32_t num_gathered,
                                              void* const* outputs, int32_t num_outputs,
                                              int64_t num_tokens, int64_t hidden,
                                              int32_t vec_per_thread, int32_t workgroups_per_cu,
                                              void* stream) {
  if (num_direct < 0 || num_direct > kProbeMaxDirect || num_gathered < 0 ||
      num_gathered > FB_MAX_TOP_K || num_outputs < 0 || num_outputs > kProbeMaxOutputs ||
      num_tokens < 0 || num_tokens > 0x7fffffffLL || hidden <= 0 || hidden % 8 != 0 ||
      hidden > FB_MAX_HIDDEN || workgroups_per_cu < 0 || workgroups_per_cu > 16 ||
      num_gathered_rows < 0)
    return FB_INVALID_ARGUMENT;
  if (vec_per_thread != 1 && vec_per_thread != 2 && vec_per_thread != 4 && vec_per_thread != 8)
    return FB_INVALID_ARGUMENT;
  if (num_tokens == 0) return FB_OK;
  if (num_direct > 0 && direct == nullptr) return FB_INVALID_ARGUMENT;
  for (int i = 0; i < num_direct; ++i)
    if (direct[i] == nullptr || ((uintptr_t)direct[i] & 15u)) return FB_INVALID_ARGUMENT;
  if (num_gathered > 0 &&
      (gathered == nullptr || gather_idx == nullptr || ((uintptr_t)gathered & 15u) ||
       num_gathered_rows == 0))
    return FB_INVALID_ARGUMENT;
  if (num_outputs > 0 && outputs == nullptr) return FB_INVALID_ARGUMENT;
  for (int d = 0; d < num_outputs; ++d)
    if (outputs[d] == nullptr || ((uintptr_t)outputs[d] & 15u)) return FB_INVALID_ARGUMENT;

  ProbeArgs a;
  memset(&a, 0, sizeof(a));
  for (int i = 0; i < num_direct; ++i) a.direct[i] = (const u32x4*)direct[i];
  a.gathered = (const u32x4*)gathered;
  a.idx = gather_idx;
  a.n_rows32 = (uint32_t)(num_gathered_rows > 0x80000000LL ? 0x80000000LL : num_gathered_rows);
  for (int d = 0; d < num_outputs; ++d) a.out[d] = (u32x4*)outputs[d];
  a.num_direct = num_direct;
  a.num_gathered = num_gathered;
  a.num_outputs = num_outputs;
  a.H8 = (int)(hidden / 8);
  const int block = ((a.H8 + vec_per_thread - 1) / vec_per_thread + 63) / 64 * 64;
  if (block > 512) return FB_INVALID_ARGUMENT;
  // the LDS reservation that holds workgroups_per_cu per CU, as the stream kernel's
  size_t lds = 0;
  if (workgroups_per_cu > 0) {
    int dev = 0, per_cu = 0, per_block = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) ==
            hipSuccess &&
        hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) ==
            hipSuccess) {
      long long share = (long long)per_cu / workgroups_per_cu - 2048;
      const long long cap = (long long)per_block - 1024;
      if (share > cap) share = cap;
      lds = share > 0 ? (size_t)share : 0;
    }
  }
  void* args[] = {&a};
  const void* fn = vec_per_thread == 1   ? reinterpret_cast<const void*>(probe_kernel<1>)
                   : vec_per_thread == 2 ? reinterpret_cast<const void*>(probe_kernel<2>)
                   : vec_per_thread == 4 ? reinterpret_cast<const void*>(probe_kernel<4>)
                                         : reinterpret_cast<const void*>(probe_kernel<8>);
  const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)num_tokens), dim3(block), args, lds,
                                       (hipStream_t)stream);
  if (e != hipSuccess) {
    t_probe_hip_error = (int)e;
    return FB_HIP_ERROR;
  }
  return FB_OK;
}

extern "C" int fused_boundary_probe_last_hip_error(void) { return t_probe_hip_error; }
