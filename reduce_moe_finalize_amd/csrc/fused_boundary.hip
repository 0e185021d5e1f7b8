// Fused post-experts boundary for MI355X (gfx950, CDNA4): partial sums + MoE
// finalize + shared expert + residual + RMSNorm in one HBM pass.
//
// What one call computes is stated in include/fused_boundary.h (with the
// passages of the sglang pull-request pages it follows).  This file holds the
// kernel and the C-ABI launcher.
//
// Design (bandwidth- and latency-bound, no matrix cores: nothing here is a
// contraction):
//  * A row of H bf16 values is split into 16-byte vectors of 8 elements.  A
//    workgroup of `block` threads owns `block * VPT` consecutive vectors of one
//    row (VPT = vectors per thread); consecutive lanes read consecutive 16-byte
//    vectors, so every source row streams through fully coalesced 128-bit loads.
//  * Sources are visited in the fixed order partials, expert slots, shared,
//    residual.  They are fetched G at a time (G*VPT independent 128-bit loads in
//    flight per lane) and then added in order, in fp32 registers.
//  * The routing metadata of a row (K indices and weights) is loaded once per
//    wave into lanes 0..K-1 and broadcast with readlane, so the expert-row
//    address of slot k is wave-uniform and costs no extra memory round trip.
//  * Sum of squares: lane partials -> wave butterfly -> LDS across waves (fixed
//    order) -> for split rows, a per-row slot array in the workspace.
//  * Split rows (small T): each of a row's `split` workgroups publishes its sum
//    of squares as one 64-bit word {epoch, value} with an agent-scope atomic
//    store and polls its siblings' words until all carry the current epoch.
//    The value rides in the same word as its epoch, so no fence is needed
//    between data and flag.  The epoch lives in the workspace header and is
//    advanced by the last workgroup of the grid, so the protocol needs no host
//    state and is safe under graph replay.  Siblings are summed in slot order:
//    results are deterministic and identical across the row's workgroups.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "fused_boundary.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr uint32_t kSpinLimit = 1u << 20;  // about a second: reached only if siblings never run
constexpr size_t kWsHeaderBytes = 256;     // status, epoch, done counter

// Workspace header words.
constexpr int kHdrStatus = 0;
constexpr int kHdrEpoch = 1;
constexpr int kHdrDone = 2;

struct KArgs {
  const u32x4* partials[FB_MAX_PARTIALS];
  const u32x4* expert;
  const int32_t* idx;
  const float* weights;
  const u32x4* shared;
  const float* gate;
  const u32x4* resid_in;
  const u32x4* gamma;
  u32x4* normed;
  u32x4* resid_out;
  unsigned long long* slots;
  uint32_t* hdr;
  long long n_rows;
  int R;
  int K;
  int has_shared;
  int H8;
  int split;
  float hidden;
  float weight_bias;
  float eps;
};

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16x2, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ int readlane_i(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}
__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

template <int VPT>
struct LaunchBound {
  static constexpr int value = VPT <= 2 ? 1024 : (VPT == 4 ? 512 : 256);
};

// G sources in flight per batch: about 8 independent 16-byte loads per lane.
template <int VPT>
struct Batch {
  static constexpr int value = VPT >= 8 ? 1 : 8 / VPT;
};

template <int VPT, bool SPLIT>
__global__ void __launch_bounds__(LaunchBound<VPT>::value) boundary_kernel(const KArgs a) {
  constexpr int G = Batch<VPT>::value;
  const int B = blockDim.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  int row, s;
  if (SPLIT) {
    row = blockIdx.x / a.split;
    s = blockIdx.x - row * a.split;
  } else {
    row = blockIdx.x;
    s = 0;
  }
  const int H8 = a.H8;
  const int vbase = s * B * VPT + tid;
  const size_t roff = (size_t)row * (size_t)H8;

  // Routing metadata first: the expert gathers depend on it.
  int my_idx = -1;
  float my_w = 0.0f;
  if (lane < a.K) {
    my_idx = a.idx[(size_t)row * a.K + lane];
    my_w = a.weights[(size_t)row * a.K + lane];
  }
  uint32_t epoch = 0;
  if (SPLIT) epoch = __hip_atomic_load(a.hdr + kHdrEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;

  // gamma + weight_bias for this thread's vectors (L2-resident across rows).
  u32x4 gam[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int v = vbase + j * B;
    gam[j] = v < H8 ? a.gamma[v] : u32x4{0u, 0u, 0u, 0u};
  }

  float sh_scale = 1.0f;
  if (a.has_shared && a.gate != nullptr) {
    const double g = (double)a.gate[row];
    sh_scale = (float)(1.0 / (1.0 + exp(-g)));
  }

  float acc[VPT][8];
#pragma unroll
  for (int j = 0; j < VPT; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;

  const int n_exp_end = a.R + a.K;
  const int nsrc = n_exp_end + a.has_shared + 1;
  for (int i0 = 0; i0 < nsrc; i0 += G) {
    u32x4 buf[G][VPT];
    float scale[G];
    bool mul[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int i = i0 + g;
      const u32x4* base = nullptr;
      float sc = 1.0f;
      bool m = false;
      if (i < a.R) {
        base = a.partials[i] + roff;
      } else if (i < n_exp_end) {
        const int k = i - a.R;
        const int e = readlane_i(my_idx, k);
        if (e >= 0 && (long long)e < a.n_rows) {
          base = a.expert + (size_t)e * (size_t)H8;
          sc = readlane_f(my_w, k);
          m = true;
        }
      } else if (i < nsrc - 1) {
        base = a.shared + roff;
        sc = sh_scale;
        m = a.gate != nullptr;
      } else if (i == nsrc - 1) {
        base = a.resid_in + roff;
      }
      scale[g] = sc;
      mul[g] = m;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int v = vbase + j * B;
        buf[g][j] = (base != nullptr && v < H8) ? base[v] : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (i0 + g < nsrc) {
        const float sc = scale[g];
        const bool m = mul[g];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float f0 = lo_bf16(buf[g][j][q]);
            const float f1 = hi_bf16(buf[g][j][q]);
            if (m) {
              // product rounded to fp32, then added: no contraction (-ffp-contract=off)
              const float p0 = sc * f0;
              const float p1 = sc * f1;
              acc[j][2 * q] = acc[j][2 * q] + p0;
              acc[j][2 * q + 1] = acc[j][2 * q + 1] + p1;
            } else {
              acc[j][2 * q] = acc[j][2 * q] + f0;
              acc[j][2 * q + 1] = acc[j][2 * q + 1] + f1;
            }
          }
        }
      }
    }
  }

  // Residual out (exact bf16 of the fp32 sum) and the lane's sum of squares.
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int v = vbase + j * B;
    if (v < H8) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[j][2 * q], acc[j][2 * q + 1]);
      a.resid_out[roff + v] = o;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(acc[j][e], acc[j][e], ss);
    }
  }

  __shared__ float red[1024 / kWave];
  __shared__ float row_total;
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  float tot = 0.0f;
  const int nw = B / kWave;
  for (int w = 0; w < nw; ++w) tot += red[w];

  if (SPLIT) {
    if (wave == 0) {
      const int sp = a.split;
      unsigned long long* rs = a.slots + (size_t)row * (size_t)sp;
      if (lane == 0) {
        const unsigned long long word = ((unsigned long long)epoch << 32) | __float_as_uint(tot);
        __hip_atomic_store(rs + s, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      float part = 0.0f;
      uint32_t spins = 0;
      bool timed_out = false;
      for (;;) {
        int ok = 1;
        if (lane < sp) {
          const unsigned long long w =
              __hip_atomic_load(rs + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = (uint32_t)(w >> 32) == epoch;
          part = __uint_as_float((uint32_t)w);
        }
        if (__all(ok)) break;
        if (++spins > kSpinLimit) {
          timed_out = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      float t2 = 0.0f;
      for (int l = 0; l < sp; ++l) t2 += readlane_f(part, l);
      if (timed_out) {
        t2 = __uint_as_float(0x7fc00000u);
        if (lane == 0)
          __hip_atomic_fetch_or(a.hdr + kHdrStatus, FB_WS_STATUS_WAIT_TIMEOUT, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
      }
      if (lane == 0) row_total = t2;
    }
    __syncthreads();
    tot = row_total;
  }

  const float r = rsqrtf(tot / a.hidden + a.eps);
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int v = vbase + j * B;
    if (v < H8) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float g0 = lo_bf16(gam[j][q]) + a.weight_bias;
        const float g1 = hi_bf16(gam[j][q]) + a.weight_bias;
        o[q] = pack_bf16x2((acc[j][2 * q] * r) * g0, (acc[j][2 * q + 1] * r) * g1);
      }
      a.normed[roff + v] = o;
    }
  }

  if (SPLIT && tid == 0) {
    // Last workgroup of the grid advances the epoch for the next call.
    const uint32_t old =
        __hip_atomic_fetch_add(a.hdr + kHdrDone, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (old == gridDim.x - 1) {
      __hip_atomic_store(a.hdr + kHdrDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.hdr + kHdrEpoch, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ----------------------------------------------------------------- host side

thread_local int t_last_hip_error = 0;
thread_local bool t_override_set = false;
thread_local fused_boundary_plan t_override = {0, 0, 0, 0};

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_cus[kMaxDevices];

int device_cus(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(g_dev_once[dev], [dev] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_dev_cus[dev] = n;
  });
  return g_dev_cus[dev];
}

int launch_bound(int vpt) { return vpt <= 2 ? 1024 : (vpt == 4 ? 512 : 256); }
bool vpt_ok(int vpt) { return vpt == 1 || vpt == 2 || vpt == 4 || vpt == 8; }
int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }
int round_up64(int x) { return (x + kWave - 1) / kWave * kWave; }

size_t ws_needed(long long T, int split) {
  return split <= 1 ? 0 : kWsHeaderBytes + (size_t)T * (size_t)split * 8u;
}

// Whole-row plan: fewest idle lanes, then fewer vectors per thread.
void whole_row(int H8, int* block, int* vpt) {
  int best_b = 0, best_v = 0;
  long long best_waste = -1;
  const int cands[4] = {2, 1, 4, 8};
  for (int c = 0; c < 4; ++c) {
    const int v = cands[c];
    const int b = round_up64(ceil_div(H8, v));
    if (b > launch_bound(v)) continue;
    const long long waste = (long long)b * v - H8;
    if (best_waste < 0 || waste < best_waste) {
      best_waste = waste;
      best_b = b;
      best_v = v;
    }
  }
  *block = best_b;
  *vpt = best_v;
}

// Automatic plan.  Large T: one workgroup per row.  Small T (fewer rows than
// about two per CU) with a workspace: split rows so that about 2 workgroups per
// CU are busy, one vector per lane.
void auto_plan(long long T, int H8, size_t ws_bytes, int cus, fused_boundary_plan* p) {
  int block = 0, vpt = 0;
  whole_row(H8, &block, &vpt);
  int split = 1;
  const long long target = 2LL * cus;
  if (T < target && H8 > kWave) {
    int want = ceil_div(target, T);
    if (want > FB_MAX_SPLIT) want = FB_MAX_SPLIT;
    if (want > 1) {
      int b = round_up64(ceil_div(H8, want));
      if (b > 1024) b = 1024;
      const int sp = ceil_div(H8, b);
      if (sp > 1 && sp <= FB_MAX_SPLIT && ws_needed(T, sp) <= ws_bytes) {
        block = b;
        vpt = 1;
        split = sp;
      }
    }
  }
  p->block = block;
  p->vec_per_thread = vpt;
  p->split = split;
  p->grid = (int)(T * split);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Call {
  const void* const* partials;
  int R;
  const void* expert;
  long long N;
  const int32_t* idx;
  const float* weights;
  int K;
  const void* shared;
  const float* gate;
  const void* resid_in;
  const void* gamma;
  float weight_bias;
  float eps;
  long long T;
  long long H;
  void* normed;
  void* resid_out;
  void* ws;
  size_t ws_bytes;
  void* stream;
};

int validate(const Call& c, bool finalize) {
  // Sizes and scalars first; with no tokens nothing is read or written, so the
  // [T, ...] pointers may be NULL (zero-size buffers).
  if (c.R < (finalize ? 0 : 1) || c.R > FB_MAX_PARTIALS) return FB_INVALID_ARGUMENT;
  if (c.T < 0 || c.T > 0x7fffffffLL || c.H <= 0) return FB_INVALID_ARGUMENT;
  if (!isfinite(c.eps) || c.eps < 0.0f || !isfinite(c.weight_bias)) return FB_INVALID_ARGUMENT;
  if (finalize && (c.K < 1 || c.K > FB_MAX_TOP_K || c.N < 0)) return FB_INVALID_ARGUMENT;
  if (c.T == 0) return (c.H % 8 != 0 || c.H > FB_MAX_HIDDEN) ? FB_DECLINED : FB_OK;
  if (c.R > 0 && c.partials == nullptr) return FB_INVALID_ARGUMENT;
  for (int r = 0; r < c.R; ++r)
    if (c.partials[r] == nullptr) return FB_INVALID_ARGUMENT;
  if (c.resid_in == nullptr || c.gamma == nullptr || c.normed == nullptr || c.resid_out == nullptr)
    return FB_INVALID_ARGUMENT;
  if (finalize) {
    if (c.idx == nullptr || c.weights == nullptr) return FB_INVALID_ARGUMENT;
    if (c.N > 0 && c.expert == nullptr) return FB_INVALID_ARGUMENT;
    if (((uintptr_t)c.idx & 3u) || ((uintptr_t)c.weights & 3u)) return FB_INVALID_ARGUMENT;
    if (c.gate != nullptr && ((uintptr_t)c.gate & 3u)) return FB_INVALID_ARGUMENT;
  }
  if (c.ws != nullptr && ((uintptr_t)c.ws & 15u)) return FB_INVALID_ARGUMENT;

  const size_t row_bytes = (size_t)c.H * 2u;
  const size_t act = (size_t)c.T * row_bytes;
  // outputs may not overlap each other, any input, or the workspace
  const void* outs[2] = {c.normed, c.resid_out};
  for (int o = 0; o < 2; ++o) {
    for (int r = 0; r < c.R; ++r)
      if (overlaps(outs[o], act, c.partials[r], act)) return FB_INVALID_ARGUMENT;
    if (overlaps(outs[o], act, c.gamma, row_bytes)) return FB_INVALID_ARGUMENT;
    if (overlaps(outs[o], act, c.ws, c.ws_bytes)) return FB_INVALID_ARGUMENT;
    if (finalize) {
      const size_t kb = (size_t)c.T * (size_t)c.K * 4u;
      if (overlaps(outs[o], act, c.expert, (size_t)c.N * row_bytes)) return FB_INVALID_ARGUMENT;
      if (overlaps(outs[o], act, c.idx, kb) || overlaps(outs[o], act, c.weights, kb))
        return FB_INVALID_ARGUMENT;
      if (c.shared != nullptr && overlaps(outs[o], act, c.shared, act)) return FB_INVALID_ARGUMENT;
      if (c.shared != nullptr && c.gate != nullptr &&
          overlaps(outs[o], act, c.gate, (size_t)c.T * 4u))
        return FB_INVALID_ARGUMENT;
    }
  }
  if (overlaps(c.normed, act, c.resid_out, act)) return FB_INVALID_ARGUMENT;
  if (overlaps(c.normed, act, c.resid_in, act)) return FB_INVALID_ARGUMENT;
  if (c.resid_out != c.resid_in && overlaps(c.resid_out, act, c.resid_in, act))
    return FB_INVALID_ARGUMENT;

  // Valid but not taken: shape or alignment outside what the kernel streams.
  if (c.H % 8 != 0 || c.H > FB_MAX_HIDDEN) return FB_DECLINED;
  for (int r = 0; r < c.R; ++r)
    if (!aligned16(c.partials[r])) return FB_DECLINED;
  if (!aligned16(c.resid_in) || !aligned16(c.gamma) || !aligned16(c.normed) ||
      !aligned16(c.resid_out))
    return FB_DECLINED;
  if (finalize && c.expert != nullptr && !aligned16(c.expert)) return FB_DECLINED;
  if (finalize && c.shared != nullptr && !aligned16(c.shared)) return FB_DECLINED;
  return FB_OK;
}

int resolve_plan(long long T, int H8, size_t ws_bytes, fused_boundary_plan* p) {
  if (t_override_set) {
    p->block = t_override.block;
    p->vec_per_thread = t_override.vec_per_thread;
    p->split = ceil_div(H8, (long long)p->block * p->vec_per_thread);
    if (p->split > FB_MAX_SPLIT) return FB_INVALID_ARGUMENT;
    if (p->split > 1 && ws_needed(T, p->split) > ws_bytes) return FB_INVALID_ARGUMENT;
    if ((long long)T * p->split > 0x7fffffffLL) return FB_INVALID_ARGUMENT;
    p->grid = (int)(T * p->split);
    return FB_OK;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  auto_plan(T, H8, ws_bytes, device_cus(dev), p);
  return FB_OK;
}

template <int VPT>
hipError_t launch_vpt(const KArgs& k, const fused_boundary_plan& p, hipStream_t st) {
  if (p.split > 1)
    hipLaunchKernelGGL((boundary_kernel<VPT, true>), dim3(p.grid), dim3(p.block), 0, st, k);
  else
    hipLaunchKernelGGL((boundary_kernel<VPT, false>), dim3(p.grid), dim3(p.block), 0, st, k);
  return hipGetLastError();
}

int run(const Call& c, bool finalize) {
  const int v = validate(c, finalize);
  if (v != FB_OK) return v;
  if (c.T == 0) return FB_OK;
  const int H8 = (int)(c.H / 8);
  fused_boundary_plan p;
  const int pr = resolve_plan(c.T, H8, c.ws == nullptr ? 0 : c.ws_bytes, &p);
  if (pr != FB_OK) return pr;

  KArgs k;
  memset(&k, 0, sizeof(k));
  for (int r = 0; r < c.R; ++r) k.partials[r] = (const u32x4*)c.partials[r];
  k.R = c.R;
  if (finalize) {
    k.expert = (const u32x4*)c.expert;
    k.idx = c.idx;
    k.weights = c.weights;
    k.K = c.K;
    k.n_rows = c.expert == nullptr ? 0 : c.N;
    k.shared = (const u32x4*)c.shared;
    k.has_shared = c.shared != nullptr ? 1 : 0;
    k.gate = c.shared != nullptr ? c.gate : nullptr;
  }
  k.resid_in = (const u32x4*)c.resid_in;
  k.gamma = (const u32x4*)c.gamma;
  k.normed = (u32x4*)c.normed;
  k.resid_out = (u32x4*)c.resid_out;
  if (p.split > 1) {
    k.hdr = (uint32_t*)c.ws;
    k.slots = (unsigned long long*)((char*)c.ws + kWsHeaderBytes);
  }
  k.H8 = H8;
  k.split = p.split;
  k.hidden = (float)c.H;
  k.weight_bias = c.weight_bias;
  k.eps = c.eps;

  hipStream_t st = (hipStream_t)c.stream;
  hipError_t e;
  switch (p.vec_per_thread) {
    case 1: e = launch_vpt<1>(k, p, st); break;
    case 2: e = launch_vpt<2>(k, p, st); break;
    case 4: e = launch_vpt<4>(k, p, st); break;
    case 8: e = launch_vpt<8>(k, p, st); break;
    default: return FB_INVALID_ARGUMENT;
  }
  if (e != hipSuccess) {
    t_last_hip_error = (int)e;
    return FB_HIP_ERROR;
  }
  return FB_OK;
}

}  // namespace

extern "C" {

int fused_reduce_rmsnorm(const void* const* partials, int32_t num_partials,
                         const void* residual_in, const void* gamma, float weight_bias,
                         float eps, int64_t num_tokens, int64_t hidden, void* normed_out,
                         void* residual_out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  Call c;
  memset(&c, 0, sizeof(c));
  c.partials = partials;
  c.R = num_partials;
  c.resid_in = residual_in;
  c.gamma = gamma;
  c.weight_bias = weight_bias;
  c.eps = eps;
  c.T = num_tokens;
  c.H = hidden;
  c.normed = normed_out;
  c.resid_out = residual_out;
  c.ws = workspace;
  c.ws_bytes = workspace == nullptr ? 0 : workspace_bytes;
  c.stream = stream;
  return run(c, false);
}

int fused_moe_finalize_rmsnorm(const void* const* partials, int32_t num_partials,
                               const void* expert_out, int64_t num_expanded_rows,
                               const int32_t* expanded_row_idx, const float* topk_weights,
                               int32_t top_k, const void* shared_out,
                               const float* shared_gate_logits, const void* residual_in,
                               const void* gamma, float weight_bias, float eps,
                               int64_t num_tokens, int64_t hidden, void* normed_out,
                               void* residual_out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  Call c;
  memset(&c, 0, sizeof(c));
  c.partials = partials;
  c.R = num_partials;
  c.expert = expert_out;
  c.N = num_expanded_rows;
  c.idx = expanded_row_idx;
  c.weights = topk_weights;
  c.K = top_k;
  c.shared = shared_out;
  c.gate = shared_gate_logits;
  c.resid_in = residual_in;
  c.gamma = gamma;
  c.weight_bias = weight_bias;
  c.eps = eps;
  c.T = num_tokens;
  c.H = hidden;
  c.normed = normed_out;
  c.resid_out = residual_out;
  c.ws = workspace;
  c.ws_bytes = workspace == nullptr ? 0 : workspace_bytes;
  c.stream = stream;
  return run(c, true);
}

size_t fused_boundary_workspace_bytes(int64_t num_tokens, int64_t hidden) {
  if (num_tokens < 0 || hidden < 0) return 0;
  return kWsHeaderBytes + (size_t)num_tokens * FB_MAX_SPLIT * 8u;
}

const char* fused_boundary_status_string(int status) {
  switch (status) {
    case FB_OK: return "ok";
    case FB_INVALID_ARGUMENT: return "invalid argument";
    case FB_DECLINED: return "declined: shape or alignment not supported by the fused kernel";
    case FB_HIP_ERROR: return "HIP error at launch";
    default: return "unknown status";
  }
}

int fused_boundary_last_hip_error(void) { return t_last_hip_error; }

int fused_boundary_get_plan(int64_t num_tokens, int64_t hidden, size_t workspace_bytes,
                            fused_boundary_plan* plan) {
  if (plan == nullptr || num_tokens < 0 || num_tokens > 0x7fffffffLL || hidden <= 0)
    return FB_INVALID_ARGUMENT;
  if (hidden % 8 != 0 || hidden > FB_MAX_HIDDEN) return FB_DECLINED;
  return resolve_plan(num_tokens, (int)(hidden / 8), workspace_bytes, plan);
}

int fused_boundary_set_plan_override(const fused_boundary_plan* plan) {
  if (plan == nullptr) {
    t_override_set = false;
    return FB_OK;
  }
  if (!vpt_ok(plan->vec_per_thread) || plan->block < kWave || plan->block % kWave != 0 ||
      plan->block > launch_bound(plan->vec_per_thread))
    return FB_INVALID_ARGUMENT;
  t_override = *plan;
  t_override_set = true;
  return FB_OK;
}

}  // extern "C"
