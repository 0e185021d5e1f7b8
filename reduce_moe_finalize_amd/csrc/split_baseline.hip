// Split (unfused) boundary: the two-launch flow the fused kernel replaces, and
// the caller's fallback after the fused entry points decline.
//
// The pages compare the fused boundary against exactly this flow: the
// post-experts reduction (and the MoE finalize) is first materialised as a bf16
// [T, H] tensor, then a separate residual RMSNorm reads it back (sglang PR
// #37104, "fuse trailing TP all-reduce with final RMSNorm", Motivation and the
// Performance table: split baseline vs fused candidate; sglang PR #37196,
// Modifications part 2: the standalone deferred-finalize call).  When the fused
// runtime declines, the owed reduction is materialised and the ordinary norm
// runs (PR #37104, Changes).
//
//   stage 1  fused_boundary_split_sum:  y = bf16( sum_r P_r + sum_k w*E[idx] + s*S )
//            (fp32, canonical order, elementwise; no row-wide step, so any grid)
//   stage 2  fused_boundary_split_residual_rmsnorm:  x = y + X;  residual_out = bf16(x);
//            normed = bf16(x * rsqrt(mean(x^2) + eps) * (gamma + weight_bias))
//
// Both stages accept any H up to FB_MAX_HIDDEN and any 2-byte aligned
// bf16 pointer: 128-bit vector kernels when every pointer is 16-byte aligned
// and H % 8 == 0, scalar kernels otherwise.  Stage 2 on aligned shapes is the
// fused reduce entry point with one partial, which computes exactly
// (0 + y) + X and the same norm.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "fused_boundary.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;
constexpr int kWave = 64;

struct SumArgs {
  const void* partials[FB_MAX_PARTIALS];
  const void* expert;
  const int32_t* idx;
  const float* weights;
  const void* shared;
  const float* gate;
  void* out;
  uint32_t n_rows32;  // min(N, 2^31): an int32 index e is valid iff (uint32)e < this
  int R;
  int K;
  int H;       // elements per row
  int chunks;  // workgroups per row
};

__device__ __forceinline__ float bf16_at(const void* base, size_t i) {
  return __uint_as_float((uint32_t)((const uint16_t*)base)[i] << 16);
}
__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float shared_scale(const float* gate, int row) {
  if (gate == nullptr) return 1.0f;
  return (float)(1.0 / (1.0 + exp(-(double)gate[row])));
}

// acc (8 lanes of a 16-byte vector) += v, or += fl32(sc * v)
__device__ __forceinline__ void add8(float* acc, u32x4 v, float sc, bool mul) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float f0 = lo_bf16(v[q]);
    const float f1 = hi_bf16(v[q]);
    if (mul) {
      const float p0 = sc * f0;
      const float p1 = sc * f1;
      acc[2 * q] = acc[2 * q] + p0;
      acc[2 * q + 1] = acc[2 * q + 1] + p1;
    } else {
      acc[2 * q] = acc[2 * q] + f0;
      acc[2 * q + 1] = acc[2 * q + 1] + f1;
    }
  }
}

// Stage 1, 16-byte vectors: one lane per vector of 8 elements.
__global__ void __launch_bounds__(kBlock) split_sum_vec_kernel(const SumArgs a) {
  const int row = blockIdx.x / a.chunks;
  const int chunk = blockIdx.x - row * a.chunks;
  const int H8 = a.H / 8;
  const int v = chunk * kBlock + threadIdx.x;
  if (v >= H8) return;
  const size_t off = (size_t)row * H8 + v;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  for (int r = 0; r < a.R; ++r) add8(acc, ((const u32x4*)a.partials[r])[off], 1.0f, false);
  for (int k = 0; k < a.K; ++k) {
    const int e = a.idx[(size_t)row * a.K + k];
    if ((uint32_t)e < a.n_rows32)
      add8(acc, ((const u32x4*)a.expert)[(size_t)e * H8 + v], a.weights[(size_t)row * a.K + k], true);
  }
  if (a.shared != nullptr)
    add8(acc, ((const u32x4*)a.shared)[off], shared_scale(a.gate, row), a.gate != nullptr);
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
  ((u32x4*)a.out)[off] = o;
}

// Stage 1, scalar: one lane per element (any H, 2-byte alignment).
__global__ void __launch_bounds__(kBlock) split_sum_scalar_kernel(const SumArgs a) {
  const int row = blockIdx.x / a.chunks;
  const int chunk = blockIdx.x - row * a.chunks;
  const int h = chunk * kBlock + threadIdx.x;
  if (h >= a.H) return;
  const size_t off = (size_t)row * a.H + h;
  float acc = 0.0f;
  for (int r = 0; r < a.R; ++r) acc = acc + bf16_at(a.partials[r], off);
  for (int k = 0; k < a.K; ++k) {
    const int e = a.idx[(size_t)row * a.K + k];
    if ((uint32_t)e < a.n_rows32) {
      const float p = a.weights[(size_t)row * a.K + k] * bf16_at(a.expert, (size_t)e * a.H + h);
      acc = acc + p;
    }
  }
  if (a.shared != nullptr) {
    const float sv = bf16_at(a.shared, off);
    const float p = a.gate != nullptr ? shared_scale(a.gate, row) * sv : sv;
    acc = acc + p;
  }
  ((uint16_t*)a.out)[off] = to_bf16(acc);
}

// Stage 2, scalar: one workgroup per row; each lane keeps its x values in
// registers between the two passes (so an in-place residual is read before it
// is overwritten).  H <= kBlock * kMaxPerLane.
constexpr int kMaxPerLane = FB_MAX_HIDDEN / kBlock;

__global__ void __launch_bounds__(kBlock) split_rmsnorm_scalar_kernel(
    const uint16_t* x_in, const uint16_t* res_in, const uint16_t* gamma, float wb, float eps,
    int H, uint16_t* normed, uint16_t* res_out) {
  __shared__ float red[kBlock / kWave];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t base = (size_t)row * H;
  float xr[kMaxPerLane];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    const int h = tid + j * kBlock;
    float a = 0.0f;
    if (h < H) {
      a = a + __uint_as_float((uint32_t)x_in[base + h] << 16);
      a = a + __uint_as_float((uint32_t)res_in[base + h] << 16);
      res_out[base + h] = to_bf16(a);
      ss = __builtin_fmaf(a, a, ss);
    }
    xr[j] = a;
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, kWave);
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = ss;
  __syncthreads();
  float tot = 0.0f;
  for (int w = 0; w < kBlock / kWave; ++w) tot += red[w];
  const float r = rsqrtf(tot / (float)H + eps);
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    const int h = tid + j * kBlock;
    if (h < H) {
      const float g = __uint_as_float((uint32_t)gamma[h] << 16) + wb;
      normed[base + h] = to_bf16((xr[j] * r) * g);
    }
  }
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}
bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }

thread_local int t_split_hip_error = 0;

// The status of one launch (hipLaunchKernel's own result, so an error left by an
// earlier, unrelated runtime call is not taken for this launch's).
int launch_status(hipError_t e) {
  if (e != hipSuccess) {
    t_split_hip_error = (int)e;
    return FB_HIP_ERROR;
  }
  return FB_OK;
}

hipError_t launch_sum(void (*kern)(SumArgs), dim3 g, dim3 b, hipStream_t st, SumArgs a) {
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), g, b, args, 0, st);
}

}  // namespace

extern "C" {

int fused_boundary_split_sum(const void* const* partials, int32_t num_partials,
                             const void* expert_out, int64_t num_expanded_rows,
                             const int32_t* expanded_row_idx, const float* topk_weights,
                             int32_t top_k, const void* shared_out,
                             const float* shared_gate_logits, int64_t num_tokens, int64_t hidden,
                             void* sum_out, void* stream) {
  const int64_t T = num_tokens, H = hidden;
  if (num_partials < 0 || num_partials > FB_MAX_PARTIALS || top_k < 0 || top_k > FB_MAX_TOP_K ||
      num_expanded_rows < 0 || num_expanded_rows > (1LL << 40) || T < 0 || T > 0x7fffffffLL ||
      H <= 0)
    return FB_INVALID_ARGUMENT;
  if (H > FB_MAX_HIDDEN) return FB_DECLINED;
  if (T == 0) return FB_OK;
  if (sum_out == nullptr || (num_partials > 0 && partials == nullptr)) return FB_INVALID_ARGUMENT;
  for (int r = 0; r < num_partials; ++r)
    if (partials[r] == nullptr || !aligned(partials[r], 2)) return FB_INVALID_ARGUMENT;
  if (top_k > 0) {
    if (expanded_row_idx == nullptr || topk_weights == nullptr) return FB_INVALID_ARGUMENT;
    if (num_expanded_rows > 0 && (expert_out == nullptr || !aligned(expert_out, 2)))
      return FB_INVALID_ARGUMENT;
    if (!aligned(expanded_row_idx, 4) || !aligned(topk_weights, 4)) return FB_INVALID_ARGUMENT;
  }
  if (shared_out != nullptr && !aligned(shared_out, 2)) return FB_INVALID_ARGUMENT;
  if (shared_out != nullptr && shared_gate_logits != nullptr && !aligned(shared_gate_logits, 4))
    return FB_INVALID_ARGUMENT;
  if (!aligned(sum_out, 2)) return FB_INVALID_ARGUMENT;
  const size_t act = (size_t)T * (size_t)H * 2u;
  for (int r = 0; r < num_partials; ++r)
    if (overlaps(sum_out, act, partials[r], act)) return FB_INVALID_ARGUMENT;
  if (top_k > 0) {
    const size_t kb = (size_t)T * (size_t)top_k * 4u;
    if (overlaps(sum_out, act, expert_out, (size_t)num_expanded_rows * (size_t)H * 2u) ||
        overlaps(sum_out, act, expanded_row_idx, kb) || overlaps(sum_out, act, topk_weights, kb))
      return FB_INVALID_ARGUMENT;
  }
  if (shared_out != nullptr && overlaps(sum_out, act, shared_out, act)) return FB_INVALID_ARGUMENT;
  if (shared_out != nullptr && shared_gate_logits != nullptr &&
      overlaps(sum_out, act, shared_gate_logits, (size_t)T * 4u))
    return FB_INVALID_ARGUMENT;

  SumArgs a;
  memset(&a, 0, sizeof(a));
  bool vec = H % 8 == 0 && aligned(sum_out, 16);
  for (int r = 0; r < num_partials; ++r) {
    a.partials[r] = partials[r];
    vec = vec && aligned(partials[r], 16);
  }
  a.R = num_partials;
  if (top_k > 0) {
    a.expert = expert_out;
    a.idx = expanded_row_idx;
    a.weights = topk_weights;
    a.K = top_k;
    const int64_t n = expert_out == nullptr ? 0 : num_expanded_rows;
    a.n_rows32 = (uint32_t)(n > 0x80000000LL ? 0x80000000LL : n);
    vec = vec && (expert_out == nullptr || aligned(expert_out, 16));
  }
  a.shared = shared_out;
  a.gate = shared_out != nullptr ? shared_gate_logits : nullptr;
  vec = vec && (shared_out == nullptr || aligned(shared_out, 16));
  a.out = sum_out;
  a.H = (int)H;
  const int64_t lanes = vec ? H / 8 : H;
  a.chunks = (int)((lanes + kBlock - 1) / kBlock);
  if (T * a.chunks > 0x7fffffffLL) return FB_INVALID_ARGUMENT;
  const dim3 grid((unsigned)(T * a.chunks)), block(kBlock);
  return launch_status(launch_sum(vec ? split_sum_vec_kernel : split_sum_scalar_kernel, grid,
                                  block, (hipStream_t)stream, a));
}

int fused_boundary_split_residual_rmsnorm(const void* x_in, const void* residual_in,
                                          const void* gamma, float weight_bias, float eps,
                                          int64_t num_tokens, int64_t hidden, void* normed_out,
                                          void* residual_out, void* stream) {
  const int64_t T = num_tokens, H = hidden;
  if (T < 0 || T > 0x7fffffffLL || H <= 0) return FB_INVALID_ARGUMENT;
  if (!isfinite(eps) || eps < 0.0f || !isfinite(weight_bias)) return FB_INVALID_ARGUMENT;
  if (H > FB_MAX_HIDDEN) return FB_DECLINED;
  if (T == 0) return FB_OK;
  if (x_in == nullptr || residual_in == nullptr || gamma == nullptr || normed_out == nullptr ||
      residual_out == nullptr)
    return FB_INVALID_ARGUMENT;
  const void* ptrs[5] = {x_in, residual_in, gamma, normed_out, residual_out};
  for (int i = 0; i < 5; ++i)
    if (!aligned(ptrs[i], 2)) return FB_INVALID_ARGUMENT;
  const size_t act = (size_t)T * (size_t)H * 2u;
  // outputs may not overlap inputs or each other; the residual may be updated in place
  if (overlaps(normed_out, act, x_in, act) || overlaps(normed_out, act, residual_in, act) ||
      overlaps(normed_out, act, gamma, (size_t)H * 2u) || overlaps(normed_out, act, residual_out, act) ||
      overlaps(residual_out, act, x_in, act) || overlaps(residual_out, act, gamma, (size_t)H * 2u) ||
      (residual_out != residual_in && overlaps(residual_out, act, residual_in, act)))
    return FB_INVALID_ARGUMENT;

  // Aligned shapes: the fused reduce entry point with the single partial y.
  const void* parts[1] = {x_in};
  const int rc = fused_reduce_rmsnorm(parts, 1, residual_in, gamma, weight_bias, eps, T, H,
                                      normed_out, residual_out, nullptr, 0, stream);
  // A failed launch is reported through this stage's own error slot too.
  if (rc == FB_HIP_ERROR) t_split_hip_error = fused_boundary_last_hip_error();
  if (rc != FB_DECLINED) return rc;

  const uint16_t* x16 = (const uint16_t*)x_in;
  const uint16_t* r16 = (const uint16_t*)residual_in;
  const uint16_t* g16 = (const uint16_t*)gamma;
  int h = (int)H;
  uint16_t* n16 = (uint16_t*)normed_out;
  uint16_t* ro16 = (uint16_t*)residual_out;
  void* args[] = {&x16, &r16, &g16, &weight_bias, &eps, &h, &n16, &ro16};
  return launch_status(hipLaunchKernel(reinterpret_cast<const void*>(split_rmsnorm_scalar_kernel),
                                       dim3((unsigned)T), dim3(kBlock), args, 0,
                                       (hipStream_t)stream));
}

int fused_boundary_split_last_hip_error(void) { return t_split_hip_error; }

}  // extern "C"
