// Fused post-experts boundary for MI355X (gfx950, CDNA4): partial sums + MoE
// finalize + shared expert + residual + RMSNorm in one HBM pass.
//
// What one call computes is stated in include/fused_boundary.h (with the
// passages of the sglang pull-request pages it follows).  This file holds the
// kernels and the C-ABI launcher.
//
// The work is bandwidth-bound at large T and latency-bound at small T; nothing
// is a contraction, so no matrix cores.  Three kernels share the arithmetic:
//
//  * stream_kernel<VPT, G>   large T.  One workgroup per row; each lane owns VPT
//    16-byte vectors (8 bf16) of the row, lanes read consecutive vectors, so
//    every source row streams through coalesced 128-bit loads.  Sources are
//    fetched G at a time (G*VPT loads in flight per lane) with the nontemporal
//    hint: nothing is reused, and keeping the stream out of the caches is worth
//    about 15 % of HBM bandwidth on this part.
//  * latency_kernel<MD, ME>  small T.  One vector per lane and every source of
//    the lane in flight at once: the K routing indices first, the direct sources
//    (residual, shared, partials) next, then the expert gathers that depend on
//    the indices, so a row costs about two memory round trips.  A row may be
//    split over several workgroups (more CUs pulling at small T); they combine
//    their sums of squares through the workspace, below.
//  * balanced_kernel<MD, ME, UPW, SB>  from one to about 1.7 rows per CU.  Rows
//    are cut into 64-vector units dealt evenly over workgroups that all fit
//    on the GPU at once; a row shared by neighbouring workgroups combines its
//    parts through the same workspace protocol.  SB = 0: every source of a
//    unit in flight at once (like the latency kernel); SB > 0, the streamed
//    form: one unit per wave, sources fetched SB at a time.
//
// All visit sources in the fixed order partials, expert slots, shared,
// residual, accumulating in fp32 registers with each product rounded to fp32
// before it is added (built with -ffp-contract=off), so residual_out is the
// bf16 rounding of one well-defined fp32 sum whatever the launch shape.
//
// Routing metadata: lanes 0..K-1 of every wave load idx/w of their slot; the
// slot's row address is then broadcast with readlane, so it is wave-uniform.
//
// Split rows.  The workspace holds a 256-byte header (word 0: status) and one
// 512-byte record per token row of 64-bit slots {32-bit epoch, 32-bit value};
// slots 0..31 are in use.  Every call that splits a row leaves all 32 slots of
// the row at one epoch E.  Workgroup s of a row reads E from its own slot s at
// start (no other workgroup writes that slot during the call), computes its
// partial sum of squares, publishes {E+1, value} there with one agent-scope
// atomic store, and polls the row's slots until all carry E+1; it then sums
// them in slot order, so every workgroup of the row gets the same,
// deterministic total.  Value and epoch share one 64-bit word, so no fence
// orders data before flag.  Workgroup 0 also stamps E+1 into the slots its
// call leaves unused, so the row ends the call at E+1 in every slot, whatever
// the split of the next call, and no slot can carry the epoch a later call
// waits for before that call publishes it (the 32-bit epoch wraps).  No
// counter to advance, no host state, no fence on the normal path: the protocol
// survives graph replay, and a workgroup that runs late still reads the epoch
// of its own call.  The record layout does not depend on T or on the split, so
// one workspace serves calls of any shape.
//
// The poll is bounded.  If siblings do not all arrive in time (the GPU is held
// by other work), the workgroup sets status bit 0, makes its own part visible
// (a release fence), and takes every sibling's part that is published by now;
// the others it computes itself from the sources, with the sibling's lanes and
// in its order, which gives the same value, so the outputs are bit-identical
// to a normal call's.  A recomputed part is used only if the sibling has still
// not published after the sources were read: with the residual updated in
// place, a workgroup of a split row stores its residual only once its own part
// is visible (after a successful poll, or after that fence), so a part still
// unpublished means the residual read was the original one.  Every workgroup
// still publishes, so the row ends the call at E+1 as usual: nothing but the
// status bit outlives a time-out.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "fused_boundary.h"

// Split-row records of the allocation-free entry point: the same layout as a
// caller's workspace (256-byte header, 512 bytes per token row) for up to
// FB_NOALLOC_MAX_ROWS rows.  Static storage starts zero-filled, which is the
// state the split-row protocol needs; the protocol itself keeps it consistent
// from call to call, so nothing is ever cleared.  Host code never passes this
// name to a kernel: it resolves the array's device address once per device
// (scratch_address below) and passes that.
static __device__ __align__(256) unsigned char
    scratch[256 + (size_t)FB_NOALLOC_MAX_ROWS * 512];

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr uint32_t kSpinLimit = 1u << 20;  // about a second: reached only if siblings never run
constexpr size_t kWsHeaderBytes = 256;     // word 0: status
constexpr size_t kWsRowBytes = 512;        // 64-bit slots; 0..kMaxSplit-1 in use
constexpr int kMaxSplit = 32;  // H <= 16384 with >= 64 lanes per workgroup
constexpr long long kMaxExpandedRows = 1LL << 40;  // keeps N * row bytes far from overflow

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
  unsigned long long* rows;  // workspace row records (split rows only)
  uint32_t* status;          // workspace status word (split rows only)
  long long n_rows;          // N, rows of the expert buffer
  uint32_t n_rows32;         // min(N, 2^31): an int32 index e is valid iff (uint32)e < this
  int R;
  int K;
  int has_shared;
  int H8;     // 16-byte vectors per row
  int split;  // workgroups per row (latency kernel)
  int units_per_row;  // balanced kernel: 64-vector units per row, ceil(H8 / 64)
  int units_q;        // balanced kernel: T * units_per_row = grid * units_q + units_m
  int units_m;
  uint32_t spin_limit;  // polls before a split row gives up (0: none, give up at once)
  int resid_in_place;   // residual_out == residual_in: split rows store it after their exchange
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

__device__ __forceinline__ u32x4 load_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
// A source pointer typed as global memory (address space 1): loads through it
// stay global loads even after the pointer went through an empty asm.
typedef const __attribute__((address_space(1))) u32x4* gsrc;
__device__ __forceinline__ u32x4 load_stream(gsrc p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_stream(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// A row store with the device-scope, non-temporal cache policy (gfx950 `sc1 nt`),
// through a buffer resource over the row: the compiler's buffer-store builtin,
// so the store is scheduled and tracked like any other.  Word 3 of the
// resource selects untyped 32-bit access; `row` is wave-uniform.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kCachePolicyNt = 2;    // buffer-store aux bit: nt
constexpr int kCachePolicySc1 = 16;  // buffer-store aux bit: sc1
__device__ __forceinline__ void store_row_device_nt(u32x4* row, int H8, int v, u32x4 val) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(row, (short)0, H8 * 16, kRawBufferWord3);
  __builtin_amdgcn_raw_buffer_store_b128(val, r, v * 16, 0, kCachePolicySc1 | kCachePolicyNt);
}

// Sum over a wave64, identical in every lane.  DPP steps (lane pairs within a
// quad, quad pairs, half-row and row mirrors) leave each 16-lane row holding its
// row sum; the four row sums are then combined in a fixed order.  Commutative
// pairings make every lane of a row bit-identical, so the result is uniform.
template <int CTRL>
__device__ __forceinline__ float dpp_step(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false);
  return v + __int_as_float(moved);
}
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_step<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_step<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_step<0x141>(v);  // row_half_mirror
  v = dpp_step<0x140>(v);  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// A 64-bit value every lane holds alike, made wave-uniform (scalar).
__device__ __forceinline__ unsigned long long uniform_u64(unsigned long long v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ int readlane_i(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// acc += v (8 bf16), or acc += fl32(sc * v) when `mul`.
__device__ __forceinline__ void add8(float* acc, u32x4 v, float sc, bool mul) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float f0 = lo_bf16(v[q]);
    const float f1 = hi_bf16(v[q]);
    if (mul) {
      const float p0 = sc * f0;  // rounded to fp32, then added: no contraction
      const float p1 = sc * f1;
      acc[2 * q] = acc[2 * q] + p0;
      acc[2 * q + 1] = acc[2 * q + 1] + p1;
    } else {
      acc[2 * q] = acc[2 * q] + f0;
      acc[2 * q + 1] = acc[2 * q + 1] + f1;
    }
  }
}

__device__ __forceinline__ u32x4 pack8(const float* acc) {
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
  return o;
}

__device__ __forceinline__ u32x4 norm8(const float* acc, float r, u32x4 gam, float wb) {
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float g0 = lo_bf16(gam[q]) + wb;
    const float g1 = hi_bf16(gam[q]) + wb;
    o[q] = pack_bf16x2((acc[2 * q] * r) * g0, (acc[2 * q + 1] * r) * g1);
  }
  return o;
}

__device__ __forceinline__ float ssq8(const float* acc, float ss) {
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(acc[e], acc[e], ss);
  return ss;
}

// Shared-expert gate logit of a row, read unconditionally (an in-bounds dummy
// word when there is no gate) so the load is issued early and never branches.
__device__ __forceinline__ float gate_logit(const KArgs& a, int row) {
  const bool gated = a.has_shared && a.gate != nullptr;
  const float* src = gated ? a.gate + row : (const float*)a.gamma;
  return *src;
}

// Shared-expert scale: sigmoid of the fp32 logit evaluated in fp64, rounded once.
__device__ __forceinline__ float shared_scale(const KArgs& a, float logit) {
  if (!a.has_shared || a.gate == nullptr) return 1.0f;
  return (float)(1.0 / (1.0 + exp(-(double)logit)));
}

// Sum over the workgroup (fixed order across waves).
__device__ __forceinline__ float block_sum(float ss, float* red) {
  const int tid = threadIdx.x;
  ss = wave_sum(ss);
  if (blockDim.x == kWave) return ss;  // one wave: no LDS round trip, no barrier
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = ss;
  __syncthreads();
  float tot = 0.0f;
  const int nw = blockDim.x / kWave;
  for (int w = 0; w < nw; ++w) tot += red[w];
  return tot;
}

// The fp32 sum of one 16-byte vector of a row in the canonical order, plain
// form: partials, valid expert slots (product rounded to fp32, then added),
// shared term, residual.  The kernels' own load schedules add a masked +0 for
// skipped slots and an absent shared expert instead of branching; +0 leaves a
// sum that starts at +0 unchanged (it is never -0), so both forms give the same
// bits.  Routing values come from lanes base .. base+K-1 of (my_idx, my_w).
__device__ __forceinline__ void source_sum(const KArgs& a, size_t roff, int vc, int my_idx,
                                           float my_w, int base, float sh_scale, float* acc) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  for (int i = 0; i < a.R; ++i) add8(acc, load_stream(a.partials[i] + roff + vc), 1.0f, false);
  for (int k = 0; k < a.K; ++k) {
    const int e = readlane_i(my_idx, base + k);
    if ((uint32_t)e < a.n_rows32)
      add8(acc, load_stream(a.expert + (size_t)e * (size_t)a.H8 + vc), readlane_f(my_w, base + k),
           true);
  }
  if (a.has_shared) add8(acc, load_stream(a.shared + roff + vc), sh_scale, a.gate != nullptr);
  add8(acc, load_stream(a.resid_in + roff + vc), 1.0f, false);
}

// Whether slot `slot` carries epoch `epoch` (its sibling has published), and
// its part if so.  Every load this wave issued before has returned when the
// slot is read (a recomputed part's inputs, see the callers).  One wave: the
// same answer in every lane.
__device__ __forceinline__ bool published_part(const unsigned long long* slot, uint32_t epoch,
                                               float* part) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const unsigned long long w =
      uniform_u64(__hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  if ((uint32_t)(w >> 32) != epoch) return false;
  *part = __uint_as_float((uint32_t)w);
  return true;
}
// The same for a whole workgroup: wave 0 reads, the answer goes through LDS
// (`flag`, `val`), so every wave takes the same branch.  Called by every thread.
__device__ __forceinline__ bool published_part_wg(const unsigned long long* slot, uint32_t epoch,
                                                  float* part, int* flag, float* val) {
  if (blockDim.x == kWave) return published_part(slot, epoch, part);
  __syncthreads();  // every wave has finished with flag / val and its loads
  if (threadIdx.x < kWave) {
    float p = 0.0f;
    const bool ok = published_part(slot, epoch, &p);
    if (threadIdx.x == 0) {
      *flag = ok ? 1 : 0;
      *val = p;
    }
  }
  __syncthreads();
  if (*flag == 0) return false;
  *part = *val;
  return true;
}

template <int VPT>
struct StreamBound {
  static constexpr int value = VPT <= 2 ? 1024 : (VPT == 4 ? 512 : 256);
};

// ------------------------------------------------------------ stream kernel
template <int VPT, int G>
__global__ void __launch_bounds__(StreamBound<VPT>::value) stream_kernel(const KArgs a) {
  const int B = blockDim.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int row = blockIdx.x;
  const int H8 = a.H8;
  const size_t roff = (size_t)row * (size_t)H8;

  int my_idx = -1;
  float my_w = 0.0f;
  if (lane < a.K) {
    my_idx = a.idx[(size_t)row * a.K + lane];
    my_w = a.weights[(size_t)row * a.K + lane];
  }
  // gamma early: measured faster than loading it after the sum (A/B at T=8192:
  // 385 vs 405 us at 8 vectors per lane) although it costs a wave per SIMD.
  u32x4 gam[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int v = tid + j * B;
    gam[j] = v < H8 ? a.gamma[v] : u32x4{0u, 0u, 0u, 0u};
  }
  const float sh_scale = shared_scale(a, gate_logit(a, row));

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
        if ((uint32_t)e < a.n_rows32) {
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
        const int v = tid + j * B;
        buf[g][j] = (base != nullptr && v < H8) ? load_stream(base + v) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (i0 + g < nsrc)
#pragma unroll
        for (int j = 0; j < VPT; ++j) add8(acc[j], buf[g][j], scale[g], mul[g]);
  }

  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int v = tid + j * B;
    if (v < H8) {
      store_stream(a.resid_out + roff + v, pack8(acc[j]));
      ss = ssq8(acc[j], ss);
    }
  }
  __shared__ float red[1024 / kWave];
  const float tot = block_sum(ss, red);
  const float r = rsqrtf(tot / a.hidden + a.eps);
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int v = tid + j * B;
    if (v < H8) store_stream(a.normed + roff + v, norm8(acc[j], r, gam[j], a.weight_bias));
  }
}

// ------------------------------------------------------------ latency kernel
// MD: direct-source register slots (residual, shared, then up to MD - 2
// partials); ME: expert slots.
//
// Load order: routing indices, the direct sources, then the expert gathers
// (one wait for the indices).  Data loads are unconditional: lanes past
// the row end read a clamped, in-bounds address and missing sources read the
// residual row, and those values are discarded.  Branch-free loads keep the
// compiler's load counters exact, so no gather waits on an unrelated load.
//
// Every source sits in a fixed register slot: slot 0 the residual, slot 1 the
// shared expert, slot 2 + i partial i, so no slot is chosen at run time.  An
// absent shared expert or a skipped or unused expert slot adds +0 through a
// zero mask instead of a branch; +0 leaves the sum unchanged because the
// running sum starts at +0 and so is never -0.  (Selecting the shared and
// residual slots by a run-time R cost about 0.5 us per call at T <= 16.)
//
// DNT: the two output rows are stored with the device-scope non-temporal cache
// policy (gfx950 `sc1 nt`) instead of plain stores.  Split rows up to half a
// row per CU take it (interleaved A/B against plain stores, T = 1..128 at
// H = 6144 / 7168 / 8192, both entry points: equal or 1-9 % faster per call,
// cold, right after other work and in a graph); whole rows per workgroup do
// not (T=256: 7 % slower cold with it), nor split rows past half a row per CU
// (H=8192 top-10, T=192: 2-5 % slower outside a graph).  A run-time switch
// between the two stores cost 2-6 % at T <= 16, hence two builds.
template <int MD, int ME, int LB, bool DNT>
__global__ void __launch_bounds__(LB) latency_kernel(const KArgs a) {
  const int B = blockDim.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int sp = a.split;
  const int row = blockIdx.x / sp;
  const int s = blockIdx.x - row * sp;
  const int H8 = a.H8;
  const int v = s * B + tid;
  const bool act = v < H8;
  const int vc = act ? v : H8 - 1;  // in-bounds address for idle lanes
  const size_t roff = (size_t)row * (size_t)H8;
  const int R = a.R;
  const int K = a.K;
  const u32x4* resid_row = a.resid_in + roff;

  // Every pointer argument up front: one burst of scalar loads.
  static_assert(MD - 2 <= FB_MAX_PARTIALS, "partial slots exceed the partial count");
  const u32x4* dptr[MD];
  dptr[0] = resid_row;
  dptr[1] = a.has_shared ? a.shared + roff : resid_row;
#pragma unroll
  for (int i = 0; i < MD - 2; ++i) dptr[2 + i] = i < R ? a.partials[i] + roff : resid_row;

  // 1. routing indices and weights
  int my_idx = -1;
  float my_w = 0.0f;
  if (lane < K) {
    my_idx = a.idx[(size_t)row * K + lane];
    my_w = a.weights[(size_t)row * K + lane];
  }
  // Row epoch (split rows): the epoch in this workgroup's own slot, which no
  // other workgroup writes during the call.  Read unconditionally so its value
  // is first waited for after the sums; whole rows read a harmless in-bounds
  // word instead.  (Issued after the sources instead, an epoch read measured
  // 0.1-0.3 us slower per call.)
  unsigned long long* rec = sp > 1 ? a.rows + (size_t)row * (kWsRowBytes / 8) : nullptr;
  const unsigned long long* ep_src = sp > 1 ? rec + s : (const unsigned long long*)a.gamma;
  const unsigned long long epoch_word =
      __hip_atomic_load(ep_src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float logit = gate_logit(a, row);
  const u32x4 gam = a.gamma[vc];

  // 2. direct sources: residual, shared, partials (in flight while the
  //    indices arrive)
  u32x4 dbuf[MD];
#pragma unroll
  for (int i = 0; i < MD; ++i) dbuf[i] = load_stream(dptr[i] + vc);
  // 3. expert gathers (one wait for the indices).  Slots past K carry index -1.
  //    A skipped slot reads the residual row (in bounds) and masks it to zero;
  //    the mask goes through an empty asm so the compiler cannot turn the load
  //    into a branch, which would make its load counting conservative.
  u32x4 ebuf[ME > 0 ? ME : 1];
  float ew[ME > 0 ? ME : 1];
#pragma unroll
  for (int k = 0; k < ME; ++k) {
    const int e = readlane_i(my_idx, k);
    const bool ok = (uint32_t)e < a.n_rows32;
    const u32x4* src = ok ? a.expert + (size_t)e * (size_t)H8 : resid_row;
    uint32_t keep = ok ? 0xffffffffu : 0u;
    asm volatile("" : "+v"(keep));
    const u32x4 val = load_stream(src + vc);
    ebuf[k] = val & keep;
    ew[k] = ok ? readlane_f(my_w, k) : 0.0f;
  }
  const float sh_scale = shared_scale(a, logit);

  // 4. canonical-order sum: partials, expert slots, shared, residual
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int i = 0; i < MD - 2; ++i)
    if (i < R) add8(acc, dbuf[2 + i], 1.0f, false);
#pragma unroll
  for (int k = 0; k < ME; ++k) add8(acc, ebuf[k], ew[k], true);  // masked slot: 0 * 0 adds +0
  uint32_t keep_shared = a.has_shared ? 0xffffffffu : 0u;
  asm volatile("" : "+v"(keep_shared));
  add8(acc, dbuf[1] & keep_shared, sh_scale, a.gate != nullptr);
  add8(acc, dbuf[0], 1.0f, false);

  // An in-place residual of a split row is stored only once this workgroup's
  // part is visible to its siblings (after the exchange): a sibling that has
  // to recompute that part reads the original residual.
  const bool defer = sp > 1 && a.resid_in_place;
  float ss = 0.0f;
  if (act) {
    if (!defer) {
      if constexpr (DNT) store_row_device_nt(a.resid_out + roff, H8, v, pack8(acc));
      else a.resid_out[roff + v] = pack8(acc);
    }
    ss = ssq8(acc, ss);
  }
  __shared__ float red[1024 / kWave];
  __shared__ float row_total;
  float tot = block_sum(ss, red);

  if (sp > 1) {
    // Wave 0 exchanges with the siblings; other waves take its result through
    // LDS (a one-wave workgroup skips that round trip and both barriers).
    __shared__ int redo_s;
    const uint32_t epoch = (uint32_t)(uniform_u64(epoch_word) >> 32) + 1u;  // this call's
    bool redo = false;
    float t2 = 0.0f;
    if (wave == 0) {
      if (lane == 0) {
        const unsigned long long word = ((unsigned long long)epoch << 32) | __float_as_uint(tot);
        __hip_atomic_store(rec + s, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else if (s == 0 && lane >= sp && lane < kMaxSplit) {
        // Slots this call leaves unused take its epoch too, so every slot of the
        // row ends the call at the same epoch, whichever slot a later call's
        // workgroup reads its epoch from, and no slot can match the epoch a
        // later call waits for (the 32-bit epoch wraps).  No sibling of this
        // call reads them.
        __hip_atomic_store(rec + lane, (unsigned long long)epoch << 32, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      float part = 0.0f;
      uint32_t spins = 0;
      redo = true;
      while (spins < a.spin_limit) {
        int ok = 1;
        if (lane < sp) {
          const unsigned long long w =
              __hip_atomic_load(rec + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = (uint32_t)(w >> 32) == epoch;
          part = __uint_as_float((uint32_t)w);
        }
        if (__all(ok)) {
          redo = false;
          break;
        }
        ++spins;
        __builtin_amdgcn_s_sleep(1);
      }
      if (!redo) {
        for (int l = 0; l < sp; ++l) t2 += readlane_f(part, l);
      } else {
        if (lane == 0)
          __hip_atomic_fetch_or(a.status, FB_WS_STATUS_WAIT_TIMEOUT, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
        // Its own part is visible before it stores an in-place residual.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      }
    }
    if (B > kWave) {
      if (tid == 0) {
        redo_s = redo ? 1 : 0;
        row_total = t2;
      }
      __syncthreads();
      redo = redo_s != 0;
      t2 = row_total;
    }
    if (redo) {
      // The parts in slot order: this workgroup's own, a sibling's if it has
      // been published by now, else recomputed here from the sibling's inputs
      // with its lanes and its order (the same value).  A recomputed part is
      // kept only if the sibling has still not published after the inputs were
      // read: a sibling overwrites an in-place residual only once its part is
      // visible, so the inputs read were the original ones.
      t2 = 0.0f;
      for (int s2 = 0; s2 < sp; ++s2) {
        float p = tot;
        if (s2 != s && !published_part_wg(rec + s2, epoch, &p, &redo_s, &row_total)) {
          if (B > kWave) __syncthreads();  // red[] is reused by each block_sum
          const int v2 = s2 * B + tid;
          const bool act2 = v2 < H8;
          float acc2[8];
          source_sum(a, roff, act2 ? v2 : H8 - 1, my_idx, my_w, 0, sh_scale, acc2);
          const float p2 = block_sum(act2 ? ssq8(acc2, 0.0f) : 0.0f, red);
          if (!published_part_wg(rec + s2, epoch, &p, &redo_s, &row_total)) p = p2;
        }
        t2 += p;
      }
    }
    tot = t2;
  }

  const float r = rsqrtf(tot / a.hidden + a.eps);
  if (act) {
    if constexpr (DNT) {
      if (defer) store_row_device_nt(a.resid_out + roff, H8, v, pack8(acc));
      store_row_device_nt(a.normed + roff, H8, v, norm8(acc, r, gam, a.weight_bias));
    } else {
      if (defer) a.resid_out[roff + v] = pack8(acc);
      a.normed[roff + v] = norm8(acc, r, gam, a.weight_bias);
    }
  }
}

// ----------------------------------------------------------- balanced kernel
// Between the small-T and the streaming regimes (about 0.5 to 4 rows per CU).
// The rows are cut into units of 64 consecutive 16-byte vectors (one wave's
// worth; a row's last unit may be shorter), numbered row-major, and workgroup
// g of the G in the grid takes units [g*U/G, (g+1)*U/G).  The host launches
// one (or a few) workgroups per CU, all resident at once and held there by an
// LDS reservation, so every CU gets the same amount of work whatever T is and
// nothing waits for a later dispatch round.  Wave w of a workgroup takes the
// workgroup's units w, w + waves, ... (at most UPW), each summed like a
// latency-kernel vector (every source in flight, fixed register slots, masked
// +0 for missing terms); its sum of squares (DPP wave sum) goes to LDS, and
// both outputs of the unit are stored at the end, once the row's total is
// known.  A row's part in the workgroup is the sum of its unit sums in unit
// order.  A row inside one workgroup is finished
// there; a row shared with neighbouring workgroups (only a workgroup's first
// and last rows can be) exchanges its parts through its workspace record,
// slot = workgroup - the row's first workgroup, with the latency kernel's
// epoch protocol: no part waits on another's wait, the wave that publishes a
// shared row's part then polls that row, and a bounded wait that gives up
// takes or recomputes the other workgroups' parts exactly.
//
// SB > 0 builds the streamed form: one unit per wave, its sources fetched SB at
// a time in the canonical order (the stream kernel's loop) instead of all at
// once, so a wave needs few registers and a CU holds 32 of them.  From a
// little past one row per CU to about two, that keeps every CU equally busy
// with a moderate number of loads in flight, where whole rows leave some CUs
// twice the work of others and all-at-once units flood HBM.
constexpr int kBalMaxRows = 16;   // rows one workgroup may touch (checked on the host)
constexpr int kBalMaxWaves = 16;  // waves per workgroup

// Units are dealt as U = G * q + m: the first m workgroups take q + 1 units,
// the others q.  First unit of workgroup g, and the workgroup holding unit u.
__device__ __forceinline__ int bal_first(int g, int q, int m) { return g * q + min(g, m); }
__device__ __forceinline__ int bal_owner(int u, int q, int m) {
  const int big = m * (q + 1);
  return u < big ? u / (q + 1) : m + (u - big) / q;
}

// Lanes per workgroup each variant is built for: as many waves as the CU holds
// at the variant's register use (<= 128 VGPRs: 1024 lanes, <= 168: 768,
// else 512), so nothing spills.
constexpr int balanced_bound(int md, int me, int upw) {
  return md == 10 && me == 0   ? (upw <= 6 ? 1024 : 768)
         : md > 10 && me == 0  ? (upw <= 3 ? 1024 : (upw <= 6 ? 768 : 512))
         : md == 10 && me == 8 ? (upw <= 2 ? 1024 : (upw <= 6 ? 768 : 512))
         : md == 10            ? (upw <= 4 ? 768 : 512)
                               : 512;
}

template <int MD, int ME, int UPW, int SB>
__global__ void __launch_bounds__(SB > 0 ? 1024 : balanced_bound(MD, ME, UPW))
    balanced_kernel(const KArgs a) {
  static_assert(SB == 0 || (MD == 0 && ME == 0 && UPW == 1), "streamed form: one unit per wave");
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform: scalar unit math
  const int nw = blockDim.x / kWave;
  const int g = blockIdx.x;
  const int q = a.units_q;
  const int m = a.units_m;
  const int nu = a.units_per_row;
  const int H8 = a.H8;
  const int R = a.R;
  const int K = a.K;
  const int u_lo = bal_first(g, q, m);
  const int u_hi = bal_first(g + 1, q, m);
  const int r_lo = u_lo / nu;
  const int nrows = (u_hi - 1) / nu - r_lo + 1;

  __shared__ float upart[UPW * kBalMaxWaves];
  __shared__ float rtot[kBalMaxRows];
  __shared__ unsigned long long rep[2];  // own slots of the first and the last row

  static_assert(MD - 2 <= FB_MAX_PARTIALS, "partial slots exceed the partial count");
  gsrc pbase[MD > 2 ? MD : 2];
  pbase[0] = (gsrc)a.resid_in;
  pbase[1] = (gsrc)(a.has_shared ? a.shared : a.resid_in);
#pragma unroll
  for (int d = 0; d < MD - 2; ++d) pbase[2 + d] = (gsrc)(d < R ? a.partials[d] : a.resid_in);

  // Routing of the workgroup's rows: lane rl*K + k holds slot k of row r_lo + rl.
  int my_idx = -1;
  float my_w = 0.0f;
  if (K > 0 && lane < nrows * K) {
    const int rl = lane / K;
    const size_t o = (size_t)(r_lo + rl) * K + (lane - rl * K);
    my_idx = a.idx[o];
    my_w = a.weights[o];
  }
  // Only the first and the last row can be shared with other workgroups.
  const int r_last = r_lo + nrows - 1;
  const bool first_shared = !(r_lo * nu >= u_lo && r_lo * nu + nu <= u_hi);
  const bool last_shared = nrows > 1 && !(r_last * nu >= u_lo && r_last * nu + nu <= u_hi);

  // Epoch of a shared row: the one in this workgroup's own slot of the row
  // (lane 0: the first row, lane 1: the last; see the latency kernel).
  unsigned long long ep = 0;
  if (wave == 0 && ((lane == 0 && first_shared) || (lane == 1 && last_shared))) {
    const int row = lane == 0 ? r_lo : r_last;
    ep = __hip_atomic_load(a.rows + (size_t)row * (kWsRowBytes / 8) + (g - bal_owner(row * nu, q, m)),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // The expert base pointer in scalar registers now, while the indices are in
  // flight (left to itself the compiler re-reads it from the kernel arguments
  // right before the first gather and waits for that read there).
  gsrc ebase = (gsrc)a.expert;
  asm volatile("" : "+s"(ebase));
  float acc[UPW][8];
  u32x4 gam[UPW];
#pragma unroll
  for (int i = 0; i < UPW; ++i) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.0f;
    gam[i] = u32x4{0u, 0u, 0u, 0u};
    const int u = u_lo + wave + i * nw;
    if (u >= u_hi) continue;
    const int row = u / nu;
    const int rl = row - r_lo;
    const int v = (u - row * nu) * kWave + lane;
    const bool act = v < H8;
    const int vc = act ? v : H8 - 1;
    const size_t roff = (size_t)row * (size_t)H8;
    const gsrc resid_row = pbase[0] + roff;
    const float logit = gate_logit(a, row);
    gam[i] = a.gamma[vc];
    if constexpr (SB > 0) {
      // Streamed: the sources in canonical order, SB in flight at a time; a
      // skipped slot or an absent shared expert adds +0 (as in the stream kernel).
      const float sh_scale = shared_scale(a, logit);
      const int n_exp_end = R + K;
      const int nsrc = n_exp_end + 2;  // the shared position always counts
      for (int i0 = 0; i0 < nsrc; i0 += SB) {
        u32x4 buf[SB];
        float scale[SB];
        bool mul[SB];
#pragma unroll
        for (int j = 0; j < SB; ++j) {
          const int si = i0 + j;
          gsrc src = nullptr;
          float sc = 1.0f;
          bool scaled = false;
          if (si < R) {
            src = (gsrc)a.partials[si] + roff;
          } else if (si < n_exp_end) {
            const int k = si - R;
            const int e = readlane_i(my_idx, rl * K + k);
            if ((uint32_t)e < a.n_rows32) {
              src = ebase + (size_t)e * (size_t)H8;
              sc = readlane_f(my_w, rl * K + k);
              scaled = true;
            }
          } else if (si == n_exp_end) {
            if (a.has_shared) {
              src = pbase[1] + roff;
              sc = sh_scale;
              scaled = a.gate != nullptr;
            }
          } else if (si == n_exp_end + 1) {
            src = resid_row;
          }
          scale[j] = sc;
          mul[j] = scaled;
          buf[j] = src != nullptr ? load_stream(src + vc) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < SB; ++j)
          if (i0 + j < nsrc) add8(acc[i], buf[j], scale[j], mul[j]);
      }
    } else {
      u32x4 dbuf[MD];
#pragma unroll
      for (int d = 0; d < MD; ++d) dbuf[d] = load_stream(pbase[d] + roff + vc);
      u32x4 ebuf[ME > 0 ? ME : 1];
      float ew[ME > 0 ? ME : 1];
#pragma unroll
      for (int k = 0; k < ME; ++k) {
        const int e = readlane_i(my_idx, rl * K + k);
        const bool ok = k < K && (uint32_t)e < a.n_rows32;
        const gsrc src = ok ? ebase + (size_t)e * (size_t)H8 : resid_row;
        uint32_t keep = ok ? 0xffffffffu : 0u;
        asm volatile("" : "+v"(keep));
        const u32x4 val = load_stream(src + vc);
        ebuf[k] = val & keep;
        ew[k] = ok ? readlane_f(my_w, rl * K + k) : 0.0f;
      }
      const float sh_scale = shared_scale(a, logit);
#pragma unroll
      for (int d = 0; d < MD - 2; ++d)
        if (d < R) add8(acc[i], dbuf[2 + d], 1.0f, false);
#pragma unroll
      for (int k = 0; k < ME; ++k) add8(acc[i], ebuf[k], ew[k], true);
      uint32_t keep_shared = a.has_shared ? 0xffffffffu : 0u;
      asm volatile("" : "+v"(keep_shared));
      add8(acc[i], dbuf[1] & keep_shared, sh_scale, a.gate != nullptr);
      add8(acc[i], dbuf[0], 1.0f, false);
    }
    // residual_out is stored with normed_out after the exchange: no store is
    // then in flight when the exchange begins (the compiler waits for every
    // outstanding memory operation before the first one here), and an in-place
    // residual of a shared row is overwritten only once this workgroup's part
    // is visible (see the latency kernel)
    const float p = wave_sum(act ? ssq8(acc[i], 0.0f) : 0.0f);
    if (lane == 0) upart[u - u_lo] = p;
  }
  __syncthreads();
  // The workgroup's part of each row: its unit sums in unit order (a fixed,
  // unrolled walk over the slots, so the LDS reads issue together rather than
  // one round trip each).
  if (tid < nrows) {
    const int row = r_lo + tid;
    const int ua = max(u_lo, row * nu) - u_lo;
    const int ub = min(u_hi, row * nu + nu) - u_lo;
    float t = 0.0f;
#pragma unroll
    for (int k = 0; k < UPW * kBalMaxWaves; ++k) {
      const float x = upart[k];
      if (k >= ua && k < ub) t += x;
    }
    rtot[tid] = t;
  }
  __syncthreads();

  if (first_shared || last_shared) {
    // No wave waits before its part is out (a chain of workgroups each waiting
    // before it publishes would serialise the whole grid).
    if (wave == 0 && lane < 2) rep[lane] = ep;
    const float part_first = rtot[0];
    const float part_last = rtot[nrows - 1];
    __syncthreads();  // every wave has read rtot before the totals replace it
    const unsigned long long e_first = rep[0];
    const unsigned long long e_last = rep[1];
    // Each shared row's part goes out from the wave that then waits for the
    // row: wave 0 for the first row, wave 1 (wave 0 if alone) for the last.
    {
#pragma unroll
      for (int side = 0; side < 2; ++side) {
        const bool sh = side == 0 ? first_shared : last_shared;
        if (!sh || wave != (side == 0 || nw == 1 ? 0 : 1)) continue;
        const unsigned long long E = side == 0 ? e_first : e_last;
        const int row = side == 0 ? r_lo : r_last;
        const int g0 = bal_owner(row * nu, q, m);
        const int nslots = bal_owner(row * nu + nu - 1, q, m) - g0 + 1;
        unsigned long long* rec = a.rows + (size_t)row * (kWsRowBytes / 8);
        const uint32_t epoch = (uint32_t)(E >> 32) + 1u;
        const float part = side == 0 ? part_first : part_last;
        if (lane == 0) {
          __hip_atomic_store(rec + (g - g0), ((unsigned long long)epoch << 32) | __float_as_uint(part),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (g == g0 && lane >= nslots && lane < kMaxSplit) {
          __hip_atomic_store(rec + lane, (unsigned long long)epoch << 32, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    // The same waves wait for the rows.
#pragma unroll
    for (int side = 0; side < 2; ++side) {
      const bool sh = side == 0 ? first_shared : last_shared;
      if (!sh || wave != (side == 0 || nw == 1 ? 0 : 1)) continue;
      const int row = side == 0 ? r_lo : r_last;
      const int rl = row - r_lo;
      const unsigned long long E = side == 0 ? e_first : e_last;
      const int g0 = bal_owner(row * nu, q, m);
      const int nslots = bal_owner(row * nu + nu - 1, q, m) - g0 + 1;
      unsigned long long* rec = a.rows + (size_t)row * (kWsRowBytes / 8);
      const uint32_t epoch = (uint32_t)(E >> 32) + 1u;
      float total = 0.0f;
      float slot = 0.0f;
      uint32_t spins = 0;
      bool redo = true;
      while (spins < a.spin_limit) {
        int ok = 1;
        if (lane < nslots) {
          const unsigned long long w =
              __hip_atomic_load(rec + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = (uint32_t)(w >> 32) == epoch;
          slot = __uint_as_float((uint32_t)w);
        }
        if (__all(ok)) {
          redo = false;
          break;
        }
        ++spins;
        __builtin_amdgcn_s_sleep(1);
      }
      if (!redo) {
        for (int l = 0; l < nslots; ++l) total += readlane_f(slot, l);
      } else {
        if (lane == 0)
          __hip_atomic_fetch_or(a.status, FB_WS_STATUS_WAIT_TIMEOUT, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
        // This wave published the row's part: it is visible before any
        // in-place residual of the row is stored (after the barrier below).
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        // Every part in slot order: this workgroup's own, another's if it has
        // been published by now, else recomputed here with that workgroup's
        // units' lanes and in its order, and kept only if it is still
        // unpublished once its inputs have been read (see the latency kernel).
        const size_t roff = (size_t)row * (size_t)H8;
        const float sc = shared_scale(a, gate_logit(a, row));
        for (int s2 = 0; s2 < nslots; ++s2) {
          float p2 = side == 0 ? part_first : part_last;
          if (g0 + s2 != g && !published_part(rec + s2, epoch, &p2)) {
            const int ua = max(bal_first(g0 + s2, q, m), row * nu);
            const int ub = min(bal_first(g0 + s2 + 1, q, m), row * nu + nu);
            float r2 = 0.0f;
            for (int u = ua; u < ub; ++u) {
              const int v2 = (u - row * nu) * kWave + lane;
              const bool act2 = v2 < H8;
              float acc2[8];
              source_sum(a, roff, act2 ? v2 : H8 - 1, my_idx, my_w, rl * K, sc, acc2);
              r2 += wave_sum(act2 ? ssq8(acc2, 0.0f) : 0.0f);
            }
            if (!published_part(rec + s2, epoch, &p2)) p2 = r2;
          }
          total += p2;
        }
      }
      if (lane == 0) rtot[rl] = total;
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < UPW; ++i) {
    const int u = u_lo + wave + i * nw;
    if (u >= u_hi) continue;
    const int row = u / nu;
    const int v = (u - row * nu) * kWave + lane;
    if (v < H8) {
      const float r = rsqrtf(rtot[row - r_lo] / a.hidden + a.eps);
      u32x4* const ro = a.resid_out + (size_t)row * (size_t)H8 + v;
      u32x4* const no = a.normed + (size_t)row * (size_t)H8 + v;
      if constexpr (SB > 0) {  // streamed: nontemporal, like the stream kernel (about 1 us faster)
        store_stream(ro, pack8(acc[i]));
        store_stream(no, norm8(acc[i], r, gam[i], a.weight_bias));
      } else {
        *ro = pack8(acc[i]);
        *no = norm8(acc[i], r, gam[i], a.weight_bias);
      }
    }
  }
}

// Latency-kernel variants by (direct-source slots, expert slots, lanes per
// workgroup): R <= 8 partials without experts, up to 8 or up to 12 expert slots,
// and the general ones (any R, K) at <= 256 lanes.  Slots past R or K cost a
// load each, so the slot counts stay close to the common shapes (R = 8; top-8,
// top-10).
enum LatVariant { kLatNoExpSmall, kLatNoExpLarge, kLatK8, kLatK12, kLatLarge };

LatVariant latency_variant(int R, int K, int has_shared) {
  (void)has_shared;  // the shared expert has its own slot in every variant
  const bool few_direct = R + 2 <= 10;
  if (K == 0) return few_direct ? kLatNoExpSmall : kLatNoExpLarge;
  if (few_direct && K <= 8) return kLatK8;
  if (few_direct && K <= 12) return kLatK12;
  return kLatLarge;
}
int latency_bound(LatVariant v) {
  switch (v) {
    case kLatNoExpSmall:
    case kLatK8: return 1024;
    case kLatK12: return 512;
    default: return 256;
  }
}

// Residency.  Waves per SIMD each kernel reaches at the register count this
// source compiles to for gfx950 (512 VGPRs per SIMD lane: 8 waves up to 64
// VGPRs, 6 up to 80, 5 up to 96, 4 up to 128, 3 up to 168, 2 up to 256) and at
// its scalar registers: on MI355X a wave holds its SGPR count plus 16, rounded
// up to a multiple of 16, of 800 per SIMD (8 waves up to 79 SGPRs, 7 up to 95,
// 6 up to 111; measured with probe kernels that record their CU and the clock),
// which neither the compiler's occupancy report nor the runtime's occupancy
// query counts.  The planner never launches a split-row or balanced grid larger
// than what can be resident at once; tests/test_abi.py checks this table
// against the compiler's resource report with that SGPR rule applied, and a
// GPU test against the runtime's occupancy query.
constexpr int kBalUpw[] = {1, 2, 3, 4, 6, 8};
constexpr int kNumBalUpw = 6;
constexpr int kMaxWgPerCu = 16;  // conservative workgroup slots per CU (checked on the GPU)
// The balanced kernel's streamed form (one unit per wave, sources two at a time)
// is built once, for every R and K: its plan carries sources_per_batch =
// kBalStreamBatch and units_per_wave 1.  Its VGPRs allow 8 waves per SIMD but
// its SGPRs (88) only 7: launches that need 8 on a SIMD (two 13- to 16-wave
// workgroups per CU, four of 8 waves) fit one workgroup fewer per CU and run
// in two rounds, about twice as long.  The planner counts on 6 (two 12-wave
// workgroups per CU, the fastest shape measured).
constexpr int kBalStreamBatch = 2;
constexpr int kBalStreamWavesPerSimd = 6;

int latency_waves_per_simd(LatVariant v) {
  switch (v) {
    case kLatNoExpSmall: return 8;
    case kLatNoExpLarge: return 4;
    case kLatK8: return 4;
    case kLatK12: return 3;
    default: return 2;
  }
}

int balanced_waves_per_simd(LatVariant v, int upw) {
  //                               upw:   1  2  3  4  6  8
  static const int t[5][kNumBalUpw] = {{6, 5, 4, 4, 4, 3},   // no experts, R <= 8
                                       {4, 4, 4, 3, 3, 0},   // no experts, R <= 16
                                       {4, 4, 3, 3, 3, 2},   // K <= 8, R <= 8
                                       {3, 3, 3, 3, 2, 2},   // K <= 12, R <= 8
                                       {2, 2, 2, 2, 2, 0}};  // any R, K
  // (0: not built; 8 units per wave spill there)
  for (int i = 0; i < kNumBalUpw; ++i)
    if (kBalUpw[i] == upw) return t[v][i];
  return 0;
}

bool balanced_upw_ok(int upw) {
  for (int i = 0; i < kNumBalUpw; ++i)
    if (kBalUpw[i] == upw) return true;
  return false;
}

// Lanes per workgroup the balanced variant is built for.
int balanced_lane_bound(LatVariant v, int upw) {
  switch (v) {
    case kLatNoExpSmall: return balanced_bound(10, 0, upw);
    case kLatNoExpLarge: return balanced_bound(FB_MAX_PARTIALS + 2, 0, upw);
    case kLatK8: return balanced_bound(10, 8, upw);
    case kLatK12: return balanced_bound(10, 12, upw);
    default: return balanced_bound(FB_MAX_PARTIALS + 2, FB_MAX_TOP_K, upw);
  }
}

// Workgroups of `block` lanes a CU holds at `waves_per_simd` (4 SIMDs), within
// an optional per-CU cap.
int resident_per_cu(int waves_per_simd, int block, int cap) {
  const int wpb = (block + kWave - 1) / kWave;
  int n = std::min(kMaxWgPerCu, 4 * waves_per_simd / wpb);
  if (cap > 0) n = std::min(n, cap);
  return n;
}

// ----------------------------------------------------------------- host side

thread_local int t_last_hip_error = 0;
thread_local uint32_t t_wait_limit = 0;  // 0: kSpinLimit; FB_WAIT_NO_POLL: no poll at all
thread_local bool t_force_decline = false;
thread_local bool t_override_set = false;
thread_local fused_boundary_plan t_override = {0, 0, 0, 0, 0, 0, 0, 0};

// Per-device properties, queried once: CU count, LDS per CU, LDS per workgroup.
struct DeviceInfo {
  int cus = 256;
  int lds_per_cu = 160 * 1024;
  int lds_per_block = 64 * 1024;
};
constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
DeviceInfo g_dev[kMaxDevices];

const DeviceInfo& device_info(int dev) {
  static const DeviceInfo fallback;
  if (dev < 0 || dev >= kMaxDevices) return fallback;
  std::call_once(g_dev_once[dev], [dev] {
    DeviceInfo d;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      d.cus = n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) ==
            hipSuccess && n > 0)
      d.lds_per_cu = n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess &&
        n > 0)
      d.lds_per_block = n;
    g_dev[dev] = d;
  });
  return g_dev[dev];
}

int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  return dev;
}

// Dynamic LDS that holds a stream-kernel launch to `wg` workgroups per CU: a
// share just under 1/wg of the CU's LDS (2 KiB of slack for the kernel's own
// LDS and the allocation granularity), within the per-workgroup limit.
size_t occupancy_lds_bytes(int wg, const DeviceInfo& d) {
  if (wg <= 0) return 0;
  const long long share = (long long)d.lds_per_cu / wg - 2048;
  const long long cap = (long long)d.lds_per_block - 1024;
  const long long lds = share < cap ? share : cap;
  return lds > 0 ? (size_t)lds : 0;
}

int stream_bound(int vpt) { return vpt <= 2 ? 1024 : (vpt == 4 ? 512 : 256); }
bool pow2_upto8(int x) { return x == 1 || x == 2 || x == 4 || x == 8; }
int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }
int round_up64(int x) { return (x + kWave - 1) / kWave * kWave; }

size_t ws_needed(long long T, int split) {
  return split <= 1 ? 0 : kWsHeaderBytes + (size_t)T * kWsRowBytes;
}


// Fill in split and grid (and, for the balanced kernel, waves) for a plan's
// launch-shape fields, and check that the plan can run these sizes.
int complete_plan(long long T, int H8, size_t ws_bytes, int R, int K, int has_shared, int cus,
                  fused_boundary_plan* p) {
  if (p->block < kWave || p->block % kWave != 0) return FB_INVALID_ARGUMENT;
  if (p->workgroups_per_cu < 0 || p->workgroups_per_cu > 16) return FB_INVALID_ARGUMENT;
  const LatVariant var = latency_variant(R, K, has_shared);
  if (p->units_per_wave != 0) {  // balanced kernel
    const int upw = p->units_per_wave;
    const int wpc = p->workgroups_per_cu == 0 ? 1 : p->workgroups_per_cu;
    const bool streamed = p->sources_per_batch != 0;
    if (p->vec_per_thread != 1) return FB_INVALID_ARGUMENT;
    if (streamed ? (p->sources_per_batch != kBalStreamBatch || upw != 1)
                 : (!balanced_upw_ok(upw) || balanced_waves_per_simd(var, upw) == 0 ||
                    p->block > balanced_lane_bound(var, upw)))
      return FB_INVALID_ARGUMENT;
    const int wps = streamed ? kBalStreamWavesPerSimd : balanced_waves_per_simd(var, upw);
    const int nw = p->block / kWave;
    const int nu = ceil_div(H8, kWave);
    const long long U = T * nu;
    if (U > (1LL << 30)) return FB_INVALID_ARGUMENT;
    const long long G = std::min(U, (long long)cus * wpc);
    const long long n_max = (U + G - 1) / G, n_min = U / G;
    if ((n_max + nw - 1) / nw > upw) return FB_INVALID_ARGUMENT;  // units per wave
    const long long rows_max = (n_max + nu - 2) / nu + 1;
    if (rows_max > kBalMaxRows || rows_max * K > kWave) return FB_INVALID_ARGUMENT;
    if ((nu - 1 + n_min - 1) / n_min + 1 > kMaxSplit) return FB_INVALID_ARGUMENT;  // slots per row
    // resident at once: registers, and the LDS reservation that holds wpc per CU
    const int per_cu = resident_per_cu(wps, p->block, 0);
    const int per_cu_lds = wpc == 1 ? 2 : wpc;
    if (G > (long long)cus * std::min(per_cu, per_cu_lds)) return FB_INVALID_ARGUMENT;
    const bool any_shared = nu > 1 && (U % G != 0 || (U / G) % nu != 0);
    if (any_shared && ws_needed(T, 2) > ws_bytes) return FB_INVALID_ARGUMENT;
    p->workgroups_per_cu = wpc;
    p->split = nu;
    p->grid = (int)G;
    p->waves = (int)G * nw;
    return FB_OK;
  }
  if (p->waves != 0) return FB_INVALID_ARGUMENT;
  if (p->sources_per_batch == 0) {  // latency kernel
    if (p->vec_per_thread != 1 || p->workgroups_per_cu != 0) return FB_INVALID_ARGUMENT;
    const int lb = latency_bound(var);
    if (p->block > lb) return FB_INVALID_ARGUMENT;
    p->split = ceil_div(H8, p->block);
    if (p->split > kMaxSplit) return FB_INVALID_ARGUMENT;
    if (p->split > 1 && ws_needed(T, p->split) > ws_bytes) return FB_INVALID_ARGUMENT;
  } else {  // stream kernel: whole rows
    if (!pow2_upto8(p->vec_per_thread) || !pow2_upto8(p->sources_per_batch))
      return FB_INVALID_ARGUMENT;
    if (p->block > stream_bound(p->vec_per_thread)) return FB_INVALID_ARGUMENT;
    if ((long long)p->block * p->vec_per_thread < H8) return FB_INVALID_ARGUMENT;
    p->split = 1;
  }
  if ((long long)T * p->split > 0x7fffffffLL) return FB_INVALID_ARGUMENT;
  p->grid = (int)(T * p->split);
  return FB_OK;
}

// Split-row latency plans must be resident at once too (a sibling that waits
// for a workgroup the dispatcher has not placed yet holds its slot).
bool latency_resident(const fused_boundary_plan& q, int R, int K, int has_shared, int cus) {
  if (q.split <= 1) return true;
  const int per_cu = resident_per_cu(latency_waves_per_simd(latency_variant(R, K, has_shared)),
                                     q.block, 0);
  return (long long)q.grid <= (long long)cus * per_cu;
}

// The balanced plan for these sizes (FB_OK), if any: the fewest units per wave
// that cover the work, with workgroups of 8 waves filling each CU (12 when a
// CU holds 3 waves per SIMD) -- two to four smaller workgroups per CU measured
// 2-3 % faster cold than one of 16 waves (H=7168 top-8, T=257 / 292).
int balanced_plan(long long T, int H8, size_t ws_bytes, int R, int K, int has_shared, int cus,
                  fused_boundary_plan* p) {
  const LatVariant var = latency_variant(R, K, has_shared);
  for (int i = 0; i < kNumBalUpw; ++i) {
    const int upw = kBalUpw[i];
    const int wps = balanced_waves_per_simd(var, upw);
    if (wps == 0) continue;
    int nw = wps % 2 == 0 ? 8 : std::min(kBalMaxWaves, 4 * wps);
    nw = std::min(nw, balanced_lane_bound(var, upw) / kWave);
    const int wpc = std::max(1, 4 * wps / nw);
    fused_boundary_plan q = {nw * kWave, 1, 0, 0, 0, wpc, upw, 0};
    if (complete_plan(T, H8, ws_bytes, R, K, has_shared, cus, &q) == FB_OK) {
      *p = q;
      return FB_OK;
    }
  }
  return FB_INVALID_ARGUMENT;
}

// The balanced kernel's streamed form at 24 waves per CU: two 12-wave
// workgroups per CU, one unit per wave (FB_OK if it fits these sizes).
int streamed_plan(long long T, int H8, size_t ws_bytes, int R, int K, int has_shared, int cus,
                  fused_boundary_plan* p) {
  fused_boundary_plan q = {768, 1, 0, 0, kBalStreamBatch, 2, 1, 0};
  if (complete_plan(T, H8, ws_bytes, R, K, has_shared, cus, &q) != FB_OK) return FB_INVALID_ARGUMENT;
  *p = q;
  return FB_OK;
}

// Automatic plan, from launch-plan sweeps on MI355X (256 CUs) at H = 6144,
// 7168 and 8192 (R = 8, top-8 and top-10 with the shared expert), HIP-graph
// timing, the mid-T choices also timed cold (after a 512 MiB flush).  With
// c = number of CUs:
//  * T <= 16: latency kernel, one wave per workgroup (rows split H/512 ways),
//    both entry points (the finalize at H = 6144 / 7168 / 8192, interleaved:
//    equal or up to 0.3 us faster per call than 128 lanes cold and right after
//    other work, level in a graph; the reduce at T=16, H=7168: 4.7 us cold
//    against 4.9 with 256 lanes).
//  * T <= 32: 128 lanes per workgroup (rows split H/1024 ways), except
//    reduce-only rows wider than 7168 (at T = 24-32, H=8192: 2-5 % slower
//    than 4 ways outside the cold case; at H = 6144 / 7168 128 lanes are 4-9 %
//    faster cold than 4 ways); past 32 rows, each row split floor(c / T) ways
//    (as many as keep every row's workgroups on separate CUs: T * ways <= c),
//    so 5-7 ways at T = 33-51, 4 to T = 64, 3 to 85, 2 to 128, whole rows
//    beyond (H=7168, cold, after other work and in a graph: T = 33-48 5 ways
//    3-9 % faster than 4; T = 72-80 3 ways 4-8 % faster than 2; T=64 5 ways
//    and T=96 3 ways, which leave some CUs two workgroups, 5-25 % slower); up
//    to T = c: whole rows in one latency workgroup (split, 4 ways past 128
//    rows, only where a row exceeds the variant's lane bound).
//    More CUs pulling on few rows beats the cross-workgroup hop it costs.
//    Without a workspace: whole rows, if a row fits one latency workgroup.
//  * c < T, H = 6144..8192, 15 to 20 units (512 elements) per CU and expert
//    gathers: the balanced kernel's streamed form, one unit per wave at 24
//    waves per CU.
//  * c < T <= 1.25c with expert gathers: the balanced kernel (rows cut into
//    64-vector units dealt evenly over resident workgroups), which evens out
//    the rows that whole rows would leave to a few CUs, where rows split 4
//    ways no longer fit on the GPU at once (measurements at that branch).
//  * T <= 2c: stream kernel, 1 vector per lane and 2 sources per batch: a whole
//    row per workgroup with as many waves as the row has vectors (H=7168 top-8,
//    T=448: 25.6 us cold against 26.6 with 2 vectors per lane; H=6144: 23.0
//    against 25.2).  Rows wider than 1024 vectors take 2 vectors per lane.
//  * T <= 3c: 2 vectors per lane, 1 source per batch (H=7168 top-8, T=640:
//    33.4 us cold against 35.9 with 4 vectors per lane; H=6144: 30.2 against
//    35.3).
//  * T < 16c: 4 vectors per lane, 1 source per batch, holding about 60 KiB of
//    source rows in flight per CU (workgroups_per_cu): as many workgroups as
//    the registers allow keep more rows open at once and stream slower.
//  * T >= 16c: for H = 5120..7168, still 4 vectors per lane, now held to about
//    12 waves per CU (interleaved A/B, T=8192: H=7168 finalize 366 us with 3
//    workgroups per CU against 379 with 8 vectors per lane at 4 per CU and 400
//    with 4 vectors at 4 per CU; reduce 202.5 against 215; H=6144 T=4096 155
//    against 173; H=5120 T=8192 262 against 268).  Other widths: 8 vectors per
//    lane at about 60 KiB per CU (H=4096 and the top-10 gated H=8192 shape
//    measured 2-3 % faster so).  Always 1 source per batch (2 measured 2-4 %
//    slower at H=6144 and H=8192 and at T=4096, and 9 % slower with 4 vectors
//    per lane at H=7168, T=8192).
//  * T > 3c and H below 5120 (rows under 640 vectors): 2 vectors per lane, held
//    to about 16 waves per CU.  With 4 or 8 vectors per lane such rows leave
//    lanes idle or give each CU few waves (interleaved A/B, top-8: H=1024
//    T=16384 107.6 us against 201.4 with 8 vectors per lane; H=2048 T=8192
//    103.5 against 121.5, T=1024 23.7 against 28.9; H=4096 T=16384 426 against
//    440, T=1024 28.0 against 32.7; H=3072 even).  Rows over 1536 vectors
//    (H=16384) likewise, one 1024-lane workgroup per CU (T=4096 427 us against
//    465 with 8 vectors per lane; T=2048 213 against 219 with 4); H=12288 keeps
//    4 vectors per lane at 12 waves from 16 rows per CU on (T=4096 317 against
//    334 with 8).
void auto_plan(long long T, int H8, size_t ws_bytes, int R, int K, int has_shared, int cus,
               fused_boundary_plan* p) {
  const int lat_lb = latency_bound(latency_variant(R, K, has_shared));
  if (T <= cus) {
    int block;
    if (T <= 16) block = kWave;  // one wave: the exchange skips LDS and barriers
    else if (T <= 32) block = (K > 0 || H8 <= 896) ? 128 : round_up64(ceil_div(H8, 4));
    else block = round_up64(ceil_div(H8, std::max(1, (int)(cus / T))));  // T * ways <= c
    if (block > round_up64(H8)) block = round_up64(H8);
    // Rows wider than the variant's lanes are split; past 128 rows, 4 ways,
    // which keeps about 3 workgroups per CU where half rows would leave some
    // CUs one and others two (H=8192 top-10, T=192: 17.0 us cold against 19.8).
    if (block > lat_lb) block = T > 128 ? std::min(lat_lb, round_up64(ceil_div(H8, 4))) : lat_lb;
    fused_boundary_plan q = {block, 1, 0, 0, 0, 0, 0, 0};
    if (complete_plan(T, H8, ws_bytes, R, K, has_shared, cus, &q) == FB_OK &&
        latency_resident(q, R, K, has_shared, cus)) {
      *p = q;
      return;
    }
    if (balanced_plan(T, H8, ws_bytes, R, K, has_shared, cus, p) == FB_OK) return;
    q = {round_up64(H8), 1, 0, 0, 0, 0, 0, 0};
    if (complete_plan(T, H8, 0, R, K, has_shared, cus, &q) == FB_OK) {
      *p = q;
      return;
    }
  } else if (K > 0 && H8 >= 768 && H8 <= 1024 && T * ceil_div(H8, kWave) > 15LL * cus &&
             T * ceil_div(H8, kWave) <= 20LL * cus &&
             streamed_plan(T, H8, ws_bytes, R, K, has_shared, cus, p) == FB_OK) {
    // H = 6144..8192 with 15 to 20 units of 512 elements per CU and expert
    // gathers: the balanced kernel's streamed form (cold, 16 interleaved calls
    // against the plans below: H=7168 top-8 T = 300 / 320 / 352 17.3 / 17.9 /
    // 19.4 us against 18.7 / 18.9 / 20.0; H=8192 top-10 gated T=257 20.0
    // against 20.4, T=300 level; H=6144 T=384 18.4 against 18.8).  Below 15
    // units per CU and from 21 on it was 1-11 % slower (the same widths, T =
    // 257-512), and slower for the reduce entry at every T measured (257-438).
    // Other widths were not measured with it.
    return;
  } else if (K > 0 && T <= (long long)cus + cus / 4 &&
             balanced_plan(T, H8, ws_bytes, R, K, has_shared, cus, p) == FB_OK) {
    // Just past one row per CU with expert gathers: whole rows would leave a
    // few CUs two rows and the others one, and rows split 4 ways in the
    // latency kernel no longer fit on the GPU at once.  The balanced kernel
    // gives every CU the same share, all resident (cold, H=7168 top-8: T=257
    // 15.9 us against 16.0-16.2 split 4 ways, 15.0 against 15.4 in a graph at
    // T=292; H=6144, T=320: 16.9 against 17.8 for the best other plan; H=8192
    // top-10 gated, T=300: 22.9 against 23.0).
    return;
  }
  // Beyond 3 rows per CU the vectors per lane follow the row width: 2 for rows
  // under 640 vectors or over 1536 (H below 5120, H = 16384), otherwise 4, and
  // from 16 rows per CU on 8 for rows of 897..1024 vectors (H = 8192).
  const bool two_vec = H8 < 640 || H8 > 1536;
  const bool eight_vec = H8 > 896 && H8 <= 1024;
  int vpt = T <= 2LL * cus ? 1
          : (T <= 3LL * cus || two_vec ? 2 : (T >= 16LL * cus && eight_vec ? 8 : 4));
  const int batch = T <= 2LL * cus ? 2 : 1;
  int block = round_up64(ceil_div(H8, vpt));
  while (block > stream_bound(vpt) && vpt < 8) {
    vpt *= 2;
    block = round_up64(ceil_div(H8, vpt));
  }
  int wg = 0;
  if (vpt == 2 && T > 3LL * cus) {
    // About 16 waves per CU (16 workgroups of 1 wave at H=1024, 8 of 2 at
    // H=2048, 4 of 4 at H=4096, 1 of 16 at H=16384).
    const int waves = block / kWave;
    wg = std::min(16, std::max(1, (16 + waves / 2) / waves));
  } else if (vpt == 4 && (T >= 16LL * cus || (K == 0 && T >= 6LL * cus))) {
    // 16 or more rows per CU: about 12 waves per CU (3 workgroups at H=7168, 4
    // at H = 5120 / 6144, 2 at H=12288); the last round of workgroups no longer
    // matters.  The reduce entry (10 sources per row, not 19) takes this from 6
    // rows per CU on (cold, H=7168: T=2048 52.9 us against 55.3 with 4 per CU,
    // T=1536 39.3 against 41.0; at T=1024 it was 10-20 % slower).
    const int waves = block / kWave;
    wg = std::max(1, (12 + waves / 2) / waves);
  } else if (vpt >= 4) {
    // One source row (2H bytes) in flight per workgroup: hold about 60 KiB per
    // CU (H = 6144 / 7168 / 8192 -> 5 / 4 / 4 workgroups per CU).  With 4
    // vectors per lane there are only 3-16 rows per CU, so the last round of
    // workgroups matters: of one fewer, that many and one more per CU, the
    // count that fills its rounds best is taken, the smaller on a tie (H=7168:
    // T=1536 67.7 us with 3 per CU against 75.0 with 4; T=2560 117.2 with 5
    // against 121.1 with 4; T=3584 158.6 with 3 against 167.6 with 4; T=1024
    // and 2048 keep 4).  (Short rows: a limit above what the registers allow
    // has no effect.)
    wg = std::min(16, std::max(3, (61440 + 8 * H8) / (16 * H8)));
    if (vpt == 4) {
      const double r = (double)T / cus;  // rows per CU
      auto fill = [r](int w) { return r / (w * std::ceil(r / w)); };
      const int base = wg;
      for (int w = base - 1; w <= base + 1; ++w)
        if (fill(w) > fill(wg) + 1e-9 || (w < wg && fill(w) >= fill(wg) - 1e-9)) wg = w;
    }
  }
  *p = {block, vpt, 1, 0, batch, wg, 0, 0};
  complete_plan(T, H8, 0, R, K, has_shared, cus, p);
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
  bool noalloc;  // split rows exchange through the static scratch array
};

int validate(const Call& c, bool finalize) {
  // Sizes and scalars first; with no tokens nothing is read or written, so the
  // [T, ...] pointers may be NULL (zero-size buffers).
  if (c.R < (finalize ? 0 : 1) || c.R > FB_MAX_PARTIALS) return FB_INVALID_ARGUMENT;
  if (c.T < 0 || c.T > 0x7fffffffLL || c.H <= 0) return FB_INVALID_ARGUMENT;
  if (!isfinite(c.eps) || c.eps < 0.0f || !isfinite(c.weight_bias)) return FB_INVALID_ARGUMENT;
  if (finalize && (c.K < 1 || c.K > FB_MAX_TOP_K || c.N < 0 || c.N > kMaxExpandedRows))
    return FB_INVALID_ARGUMENT;
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
  // Wider rows than the kernels take are declined before any size arithmetic.
  if (c.H > FB_MAX_HIDDEN) return FB_DECLINED;

  const size_t row_bytes = (size_t)c.H * 2u;
  const size_t act = (size_t)c.T * row_bytes;
  const size_t kb = (size_t)c.T * (size_t)c.K * 4u;
  // Every buffer the kernel reads, with its extent, and whether it is read
  // only at the [T, H] position that the same lane later writes (a row of
  // token t, vector v), which is what makes an in-place update safe.
  const void* in_ptr[FB_MAX_PARTIALS + 7];
  size_t in_len[FB_MAX_PARTIALS + 7];
  bool in_rowwise[FB_MAX_PARTIALS + 7];
  int n_in = 0;
  auto add_in = [&](const void* p, size_t len, bool rowwise) {
    in_ptr[n_in] = p;
    in_len[n_in] = len;
    in_rowwise[n_in++] = rowwise;
  };
  for (int r = 0; r < c.R; ++r) add_in(c.partials[r], act, true);
  add_in(c.resid_in, act, true);
  add_in(c.gamma, row_bytes, false);
  if (finalize) {
    add_in(c.expert, (size_t)c.N * row_bytes, false);  // gathered at any row
    add_in(c.idx, kb, false);
    add_in(c.weights, kb, false);
    if (c.shared != nullptr) {
      add_in(c.shared, act, true);
      if (c.gate != nullptr) add_in(c.gate, (size_t)c.T * 4u, false);
    }
  }
  // Outputs may not overlap each other, the workspace or any input, except
  // that residual_out may be exactly residual_in, updating it in place (so
  // also a partial or the shared-expert buffer that is that same buffer); the
  // workspace may not overlap any input either.
  for (int i = 0; i < n_in; ++i) {
    if (in_rowwise[i] && in_ptr[i] == c.resid_in && c.resid_out == c.resid_in &&
        in_len[i] == act) {
      if (overlaps(c.normed, act, in_ptr[i], in_len[i])) return FB_INVALID_ARGUMENT;
    } else if (overlaps(c.normed, act, in_ptr[i], in_len[i]) ||
               overlaps(c.resid_out, act, in_ptr[i], in_len[i])) {
      return FB_INVALID_ARGUMENT;
    }
    if (overlaps(c.ws, c.ws_bytes, in_ptr[i], in_len[i])) return FB_INVALID_ARGUMENT;
  }
  if (overlaps(c.normed, act, c.resid_out, act)) return FB_INVALID_ARGUMENT;
  if (overlaps(c.normed, act, c.ws, c.ws_bytes) || overlaps(c.resid_out, act, c.ws, c.ws_bytes))
    return FB_INVALID_ARGUMENT;

  // Valid but not taken: shape or alignment outside what the kernels stream.
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

// Device address of this device's copy of `scratch`, resolved once per device
// with that device current (the first allocation-free call on it).  No
// allocation: the array is part of the loaded code object.
struct ScratchAddr {
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
std::once_flag g_scratch_once[kMaxDevices];
ScratchAddr g_scratch[kMaxDevices];

const ScratchAddr& scratch_address(int dev) {
  static const ScratchAddr bad = {nullptr, hipErrorInvalidDevice};
  if (dev < 0 || dev >= kMaxDevices) return bad;
  std::call_once(g_scratch_once[dev], [dev] {
    ScratchAddr a;
    a.err = hipGetSymbolAddress(&a.ptr, HIP_SYMBOL(scratch));
    if (a.err != hipSuccess) a.ptr = nullptr;
    g_scratch[dev] = a;
  });
  return g_scratch[dev];
}

int resolve_plan(long long T, int H8, size_t ws_bytes, int R, int K, int has_shared,
                 fused_boundary_plan* p) {
  const int cus = device_info(current_device()).cus;
  if (t_override_set) {
    *p = t_override;
    return complete_plan(T, H8, ws_bytes, R, K, has_shared, cus, p);
  }
  auto_plan(T, H8, ws_bytes, R, K, has_shared, cus, p);
  return FB_OK;
}

// One launch; the returned status is this launch's own (not an error left
// behind by an earlier, unrelated runtime call).
hipError_t launch_kernel(void (*kern)(KArgs), dim3 g, dim3 b, hipStream_t st, KArgs k,
                         size_t lds = 0) {
  void* args[] = {&k};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), g, b, args, lds, st);
}

template <int VPT>
hipError_t launch_stream_vpt(const KArgs& k, const fused_boundary_plan& p, hipStream_t st) {
  const dim3 g(p.grid), b(p.block);
  const size_t lds = occupancy_lds_bytes(p.workgroups_per_cu, device_info(current_device()));
  switch (p.sources_per_batch) {
    case 1: return launch_kernel(stream_kernel<VPT, 1>, g, b, st, k, lds);
    case 2: return launch_kernel(stream_kernel<VPT, 2>, g, b, st, k, lds);
    case 4: return launch_kernel(stream_kernel<VPT, 4>, g, b, st, k, lds);
    default: return launch_kernel(stream_kernel<VPT, 8>, g, b, st, k, lds);
  }
}

// Kernel entry of the latency (upw 0) or balanced kernel a launch would use.
template <int MD, int ME>
const void* balanced_fn(int upw) {
  switch (upw) {
    case 1: return reinterpret_cast<const void*>(balanced_kernel<MD, ME, 1, 0>);
    case 2: return reinterpret_cast<const void*>(balanced_kernel<MD, ME, 2, 0>);
    case 3: return reinterpret_cast<const void*>(balanced_kernel<MD, ME, 3, 0>);
    case 4: return reinterpret_cast<const void*>(balanced_kernel<MD, ME, 4, 0>);
    case 6: return reinterpret_cast<const void*>(balanced_kernel<MD, ME, 6, 0>);
    default:
      if constexpr (MD > 10) return nullptr;  // not built
      else return reinterpret_cast<const void*>(balanced_kernel<MD, ME, 8, 0>);
  }
}
const void* kernel_fn(LatVariant v, int upw, int spb) {
  if (upw > 0 && spb > 0) return reinterpret_cast<const void*>(balanced_kernel<0, 0, 1, kBalStreamBatch>);
  if (upw > 0) {
    switch (v) {
      case kLatNoExpSmall: return balanced_fn<10, 0>(upw);
      case kLatNoExpLarge: return balanced_fn<FB_MAX_PARTIALS + 2, 0>(upw);
      case kLatK8: return balanced_fn<10, 8>(upw);
      case kLatK12: return balanced_fn<10, 12>(upw);
      default: return balanced_fn<FB_MAX_PARTIALS + 2, FB_MAX_TOP_K>(upw);
    }
  }
  // the split-row build: the one whose workgroups wait for each other
  switch (v) {
    case kLatNoExpSmall: return reinterpret_cast<const void*>(latency_kernel<10, 0, 1024, true>);
    case kLatNoExpLarge:
      return reinterpret_cast<const void*>(latency_kernel<FB_MAX_PARTIALS + 2, 0, 256, true>);
    case kLatK8: return reinterpret_cast<const void*>(latency_kernel<10, 8, 1024, true>);
    case kLatK12: return reinterpret_cast<const void*>(latency_kernel<10, 12, 512, true>);
    default:
      return reinterpret_cast<const void*>(
          latency_kernel<FB_MAX_PARTIALS + 2, FB_MAX_TOP_K, 256, true>);
  }
}

template <int MD, int ME>
hipError_t launch_balanced_md(const KArgs& k, const fused_boundary_plan& p, hipStream_t st) {
  const dim3 g(p.grid), b(p.block);
  // two or more per CU: the reservation holds that many; one per CU: the
  // planner takes as many waves as a CU holds
  const size_t lds = p.workgroups_per_cu >= 2
                         ? occupancy_lds_bytes(p.workgroups_per_cu, device_info(current_device()))
                         : 0;
  switch (p.units_per_wave) {
    case 1: return launch_kernel(balanced_kernel<MD, ME, 1, 0>, g, b, st, k, lds);
    case 2: return launch_kernel(balanced_kernel<MD, ME, 2, 0>, g, b, st, k, lds);
    case 3: return launch_kernel(balanced_kernel<MD, ME, 3, 0>, g, b, st, k, lds);
    case 4: return launch_kernel(balanced_kernel<MD, ME, 4, 0>, g, b, st, k, lds);
    case 6: return launch_kernel(balanced_kernel<MD, ME, 6, 0>, g, b, st, k, lds);
    default:
      if constexpr (MD > 10) return hipErrorInvalidValue;  // not built (would spill)
      else return launch_kernel(balanced_kernel<MD, ME, 8, 0>, g, b, st, k, lds);
  }
}

template <bool DNT>
hipError_t launch_latency(const KArgs& k, const fused_boundary_plan& p, hipStream_t st) {
  const dim3 g(p.grid), b(p.block);
  switch (latency_variant(k.R, k.K, k.has_shared)) {
    case kLatNoExpSmall: return launch_kernel(latency_kernel<10, 0, 1024, DNT>, g, b, st, k);
    case kLatNoExpLarge:
      return launch_kernel(latency_kernel<FB_MAX_PARTIALS + 2, 0, 256, DNT>, g, b, st, k);
    case kLatK8: return launch_kernel(latency_kernel<10, 8, 1024, DNT>, g, b, st, k);
    case kLatK12: return launch_kernel(latency_kernel<10, 12, 512, DNT>, g, b, st, k);
    default:
      return launch_kernel(latency_kernel<FB_MAX_PARTIALS + 2, FB_MAX_TOP_K, 256, DNT>, g, b, st,
                           k);
  }
}

hipError_t launch(const KArgs& k, const fused_boundary_plan& p, hipStream_t st) {
  if (p.units_per_wave > 0 && p.sources_per_batch > 0) {  // streamed balanced kernel
    const size_t lds = p.workgroups_per_cu >= 2
                           ? occupancy_lds_bytes(p.workgroups_per_cu, device_info(current_device()))
                           : 0;
    return launch_kernel(balanced_kernel<0, 0, 1, kBalStreamBatch>, dim3(p.grid), dim3(p.block), st,
                         k, lds);
  }
  if (p.units_per_wave > 0) {
    switch (latency_variant(k.R, k.K, k.has_shared)) {
      case kLatNoExpSmall: return launch_balanced_md<10, 0>(k, p, st);
      case kLatNoExpLarge: return launch_balanced_md<FB_MAX_PARTIALS + 2, 0>(k, p, st);
      case kLatK8: return launch_balanced_md<10, 8>(k, p, st);
      case kLatK12: return launch_balanced_md<10, 12>(k, p, st);
      default: return launch_balanced_md<FB_MAX_PARTIALS + 2, FB_MAX_TOP_K>(k, p, st);
    }
  }
  if (p.sources_per_batch == 0) {
    // split rows up to half a row per CU store with the device-scope
    // non-temporal policy (see latency_kernel)
    const long long rows = p.grid / p.split;
    const bool dnt = p.split > 1 && rows <= device_info(current_device()).cus / 2;
    return dnt ? launch_latency<true>(k, p, st) : launch_latency<false>(k, p, st);
  }
  switch (p.vec_per_thread) {
    case 1: return launch_stream_vpt<1>(k, p, st);
    case 2: return launch_stream_vpt<2>(k, p, st);
    case 4: return launch_stream_vpt<4>(k, p, st);
    default: return launch_stream_vpt<8>(k, p, st);
  }
}

int run(Call c, bool finalize) {
  const int v = validate(c, finalize);
  if (v != FB_OK) return v;
  if (c.noalloc && c.T > FB_NOALLOC_MAX_ROWS) return FB_TOO_MANY_ROWS;
  if (c.T == 0) return FB_OK;
  if (t_force_decline) return FB_DECLINED;  // test hook: a decline on any valid call
  if (c.noalloc) {
    const ScratchAddr& sa = scratch_address(current_device());
    if (sa.ptr == nullptr) {
      t_last_hip_error = (int)sa.err;
      return FB_HIP_ERROR;
    }
    c.ws = sa.ptr;
    c.ws_bytes = sizeof(scratch);
  }
  const int H8 = (int)(c.H / 8);
  const int K = finalize ? c.K : 0;
  const int has_shared = (finalize && c.shared != nullptr) ? 1 : 0;
  fused_boundary_plan p;
  const int pr = resolve_plan(c.T, H8, c.ws == nullptr ? 0 : c.ws_bytes, c.R, K, has_shared, &p);
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
    k.n_rows32 = (uint32_t)(k.n_rows > 0x80000000LL ? 0x80000000LL : k.n_rows);
    k.shared = (const u32x4*)c.shared;
    k.has_shared = has_shared;
    k.gate = has_shared ? c.gate : nullptr;
  }
  k.resid_in = (const u32x4*)c.resid_in;
  k.gamma = (const u32x4*)c.gamma;
  k.normed = (u32x4*)c.normed;
  k.resid_out = (u32x4*)c.resid_out;
  const bool exchange = p.split > 1;  // split rows, or rows of several balanced units
  if (exchange) {
    k.status = (uint32_t*)c.ws;
    k.rows = (unsigned long long*)((char*)c.ws + kWsHeaderBytes);
  }
  k.H8 = H8;
  k.split = p.units_per_wave > 0 ? 1 : p.split;
  if (p.units_per_wave > 0) {
    k.units_per_row = p.split;
    const long long U = c.T * p.split;
    k.units_q = (int)(U / p.grid);
    k.units_m = (int)(U % p.grid);
  }
  k.resid_in_place = c.resid_out == c.resid_in ? 1 : 0;
  k.spin_limit = t_wait_limit == 0 ? kSpinLimit
                : (t_wait_limit == FB_WAIT_NO_POLL ? 0u : t_wait_limit);
  k.hidden = (float)c.H;
  k.weight_bias = c.weight_bias;
  k.eps = c.eps;

  const hipError_t e = launch(k, p, (hipStream_t)c.stream);
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

int fused_moe_finalize_rmsnorm_noalloc(const void* const* partials, int32_t num_partials,
                                       const void* expert_out, int64_t num_expanded_rows,
                                       const int32_t* expanded_row_idx,
                                       const float* topk_weights, int32_t top_k,
                                       const void* shared_out, const float* shared_gate_logits,
                                       const void* residual_in, const void* gamma,
                                       float weight_bias, float eps, int64_t num_tokens,
                                       int64_t hidden, void* normed_out, void* residual_out,
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
  c.stream = stream;
  c.noalloc = true;
  if (top_k == 0) return run(c, false);  // no MoE finalize: the reduce entry point's call
  c.expert = expert_out;
  c.N = num_expanded_rows;
  c.idx = expanded_row_idx;
  c.weights = topk_weights;
  c.K = top_k;
  c.shared = shared_out;
  c.gate = shared_gate_logits;
  return run(c, true);
}

size_t fused_boundary_workspace_bytes(int64_t num_tokens, int64_t hidden) {
  if (num_tokens < 0 || hidden < 0) return 0;
  return kWsHeaderBytes + (size_t)num_tokens * kWsRowBytes;
}

const char* fused_boundary_status_string(int status) {
  switch (status) {
    case FB_OK: return "ok";
    case FB_INVALID_ARGUMENT: return "invalid argument";
    case FB_DECLINED: return "declined: shape or alignment not supported by the fused kernel";
    case FB_HIP_ERROR: return "HIP error at launch";
    case FB_TOO_MANY_ROWS:
      return "num_tokens exceeds FB_NOALLOC_MAX_ROWS, the row capacity of the allocation-free "
             "entry point's static scratch (use an entry point that takes a workspace)";
    default: return "unknown status";
  }
}

int fused_boundary_last_hip_error(void) { return t_last_hip_error; }

void fused_boundary_set_wait_limit(uint32_t polls) { t_wait_limit = polls; }

int fused_boundary_resident_workgroups(int32_t num_partials, int32_t top_k,
                                       int32_t units_per_wave, int32_t sources_per_batch,
                                       int32_t block, int32_t* planned, int32_t* device) {
  if (planned == nullptr || device == nullptr || num_partials < 0 ||
      num_partials > FB_MAX_PARTIALS || top_k < 0 || top_k > FB_MAX_TOP_K || block < kWave ||
      block % kWave != 0 || block > 1024 || (units_per_wave != 0 && !balanced_upw_ok(units_per_wave)))
    return FB_INVALID_ARGUMENT;
  const bool streamed = sources_per_batch != 0;
  if (streamed && (units_per_wave != 1 || sources_per_batch != kBalStreamBatch))
    return FB_INVALID_ARGUMENT;
  const LatVariant v = latency_variant(num_partials, top_k, 1);
  if (units_per_wave == 0 && block > latency_bound(v)) return FB_INVALID_ARGUMENT;
  const int wps = streamed              ? kBalStreamWavesPerSimd
                  : units_per_wave > 0 ? balanced_waves_per_simd(v, units_per_wave)
                                       : latency_waves_per_simd(v);
  if (units_per_wave > 0 && !streamed && (wps == 0 || block > balanced_lane_bound(v, units_per_wave)))
    return FB_INVALID_ARGUMENT;
  *planned = resident_per_cu(wps, block, 0);
  int n = -1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel_fn(v, units_per_wave, sources_per_batch),
                                                   block, 0) != hipSuccess) {
    *device = -1;
    return FB_HIP_ERROR;
  }
  *device = n;
  return FB_OK;
}

void fused_boundary_set_force_decline(int on) { t_force_decline = on != 0; }

int fused_boundary_get_plan(int64_t num_tokens, int64_t hidden, int32_t num_partials,
                            int32_t top_k, int32_t has_shared, size_t workspace_bytes,
                            fused_boundary_plan* plan) {
  if (plan == nullptr || num_tokens < 0 || num_tokens > 0x7fffffffLL || hidden <= 0 ||
      num_partials < 0 || num_partials > FB_MAX_PARTIALS || top_k < 0 || top_k > FB_MAX_TOP_K)
    return FB_INVALID_ARGUMENT;
  if (hidden % 8 != 0 || hidden > FB_MAX_HIDDEN) return FB_DECLINED;
  return resolve_plan(num_tokens, (int)(hidden / 8), workspace_bytes, num_partials, top_k,
                      has_shared ? 1 : 0, plan);
}

int fused_boundary_set_plan_override(const fused_boundary_plan* plan) {
  if (plan == nullptr) {
    t_override_set = false;
    return FB_OK;
  }
  const bool balanced = plan->units_per_wave != 0;
  const bool latency = !balanced && plan->sources_per_batch == 0;
  if (plan->block < kWave || plan->block % kWave != 0 || plan->block > 1024) return FB_INVALID_ARGUMENT;
  if (plan->workgroups_per_cu < 0 || plan->workgroups_per_cu > 16) return FB_INVALID_ARGUMENT;
  if (balanced && (!balanced_upw_ok(plan->units_per_wave) || plan->vec_per_thread != 1 ||
                   (plan->sources_per_batch != 0 &&
                    (plan->sources_per_batch != kBalStreamBatch || plan->units_per_wave != 1))))
    return FB_INVALID_ARGUMENT;
  if (latency && (plan->vec_per_thread != 1 || plan->workgroups_per_cu != 0))
    return FB_INVALID_ARGUMENT;
  if (!balanced && !latency &&
      (!pow2_upto8(plan->vec_per_thread) || !pow2_upto8(plan->sources_per_batch) ||
       plan->block > stream_bound(plan->vec_per_thread)))
    return FB_INVALID_ARGUMENT;
  t_override = *plan;
  t_override_set = true;
  return FB_OK;
}

}  // extern "C"
