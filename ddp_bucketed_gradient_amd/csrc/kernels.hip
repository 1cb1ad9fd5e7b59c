// kernels.hip -- CDNA4 (gfx950) kernels and the HIP launcher of the bucketed
// gradient reducer.
//
// The reduction of one bucket ([Li] "Overlapping Computation with
// Communication"; [TP] "Internal Design", backward pass; [PDTI] §3) is the
// elementwise mean over R replicas, m = fl(fl(..fl(g_0 + g_1).. + g_{R-1}) / R),
// summed in replica order in fp32 and divided once (IEEE, nearest-even),
// written back into every replica's gradient. On one GPU the replicas sit in
// HBM, so the path is bound by HBM bandwidth: each kernel streams its bytes
// once with 128-bit accesses and does a handful of adds per element.
//
// Work decomposition: the host cuts every bucket member into segments of at
// most kSegElems (8192) elements (plan.cpp). One wavefront owns one segment;
// a workgroup of 256 threads owns four consecutive segments. Each lane moves
// v4fs at lane stride, so one instruction covers 1 KiB of contiguous memory
// per replica. An unrolled group issues all of its R x U loads before the
// first add, to keep enough bytes in flight, each under its own bound check
// so that they leave one at a time (measured faster than back to back). All
// gradient streams are non-temporal; the reduction's stores (and those of the
// bf16 accumulation and the staged copy-back) also carry device scope, which
// needs the buffer-resource form of the accesses (seg_rsrc below).
//
// Kernels
//   fused_mean_kernel   gather (pack), R-way mean and copy-back in one pass:
//                       reads R*S_b and writes R*S_b bytes per bucket.
//   fused_mean_kernel_rt  the same for a replica count known at run time
//                       (above 16), replicas in chunks of 8.
//   pack_kernel         staged step 1: R gradients -> R flat buckets.
//   mean_kernel         staged step 2: R flat buckets -> averaged bucket,
//                       grid-stride over contiguous v4fs.
//   copyback_kernel     staged step 3: averaged bucket -> R gradients.
//   accumulate_kernel   no_sync: grad (+)= float(step) for every replica.
//   fused_acc_mean_kernel  the synchronising micro-step fused into the
//                       reduction: mean of (grad + float(step)) in one pass.
//
// With used flags (unused parameters) the kernels read zeros for replicas that
// did not use a variable and skip variables no replica used (bucket views:
// write them as zeros).
//
// Occupancy: a CU runs one workgroup of these streaming kernels at a time by
// default (each workgroup reserves more than half the CU's LDS, which the
// kernels do not use). More concurrent waves per CU only add DRAM streams and
// let one CU fall behind the others; ddpb_set_workgroups_per_cu relaxes it for
// the reduction kernels when they share the GPU with a backward.
//
// Short page names are defined in core.hpp.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "core.hpp"

// Device memory of the allocation-free bindings (ddpb_bind_static): their
// pointer and segment tables and, in staged mode, their flat buckets. Every
// device that loads the library holds one copy until the process ends. Host
// code never uses this name as an address: the address of a device's copy
// comes from hipGetSymbolAddress (static_scratch_base below).
static __device__ __align__(256) unsigned char scratch[ddpb::kStaticScratchBytes];

namespace ddpb {
namespace {

constexpr int kMaxDevices = 64;

// Per device: the address of its copy of `scratch` (looked up once, with the
// device current) and the launcher whose tables it holds now.
std::mutex g_scratch_mu;
char* g_scratch_base[kMaxDevices] = {};
const void* g_scratch_owner[kMaxDevices] = {};

int static_scratch_base(int device, char** base, std::string* err) {
  if (device < 0 || device >= kMaxDevices) {
    *err = "bind_static: device ordinal out of range";
    return kErrArg;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_base[device] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      *err = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
      return kErrHip;
    }
    g_scratch_base[device] = static_cast<char*>(p);
  }
  *base = g_scratch_base[device];
  return kOk;
}

constexpr int kWavesPerBlock = 4;
constexpr int kBlock = 64 * kWavesPerBlock;
constexpr int kStepSlots = 8;

#define HIP_OK(expr, what)                                                        \
  do {                                                                            \
    hipError_t e_ = (expr);                                                       \
    if (e_ != hipSuccess) {                                                       \
      *err = std::string(what) + ": " + hipGetErrorString(e_);                    \
      return kErrHip;                                                             \
    }                                                                             \
  } while (0)

// ---------------------------------------------------------------------------
// device helpers

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Gradient pointers come from a device table, so the compiler cannot tell
// they address global memory and would emit flat accesses (which share a
// counter with scalar loads and force full waits). All gradient traffic goes
// through address-space-1 pointers to native 4-wide vectors instead, which
// become global_load_dwordx4 / global_store_dwordx4.
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) float gfloat;
typedef __attribute__((address_space(1))) v4f gv4f;

__device__ __forceinline__ gfloat* G(float* p) { return (gfloat*)p; }
__device__ __forceinline__ const gfloat* G(const float* p) { return (const gfloat*)p; }
__device__ __forceinline__ v4f ld4(const float* p) { return *(const gv4f*)p; }
__device__ __forceinline__ void st4(float* p, v4f v) { *(gv4f*)p = v; }
// Streaming variants: every gradient byte is touched exactly once per launch,
// so the data are marked non-temporal and do not displace other kernels'
// working sets in L2 and the Infinity Cache.
__device__ __forceinline__ v4f ld4s(const float* p) { return __builtin_nontemporal_load((const gv4f*)p); }
__device__ __forceinline__ void st4s(float* p, v4f v) { __builtin_nontemporal_store(v, (gv4f*)p); }

// The reduction kernels address one wavefront's segment of one replica (a
// wave-uniform base, at most 32 KiB) through a buffer resource, which lets the
// stores carry device scope (sc1) beside the non-temporal hint: on gfx950 the
// BERT-large sync (R = 8, cap 25 MiB) ran 1.0 % faster with such stores than
// with plain non-temporal ones (5,803-5,806 against 5,740-5,749 GB/s, three
// interleaved runs each on one box; 5,754-5,768 against 5,698-5,706 on
// another). Device scope without the hint was 3.4 % slower, sc0 with it
// changed nothing, and none of the policy bits changed anything on the loads,
// which stay plain non-temporal.
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
constexpr int kPolicyNT = 2;               // cache-policy operand: nt
constexpr int kPolicyDeviceNT = 2 | 16;    // nt and sc1
// Word 3 of a gfx9 buffer resource: data format 32 (bits 18:15 = 4), every
// other field zero (no swizzle, no stride: raw byte offsets, bounded by the
// record count in bytes; accesses beyond it read zero and write nothing).
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t seg_rsrc(const float* p, int bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  void* base = reinterpret_cast<void*>((static_cast<uintptr_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, kRsrcWord3);
}
__device__ __forceinline__ v4f bld4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kPolicyNT));
}
__device__ __forceinline__ void bst4(__amdgpu_buffer_rsrc_t r, int byte_off, v4f v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, byte_off, 0, kPolicyDeviceNT);
}

typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) v2u gv2u;

template <int R>
__device__ __forceinline__ float finish(float acc, float scale) {
  // Power-of-two R: 1/R is exact, so the product is the correctly rounded
  // quotient. Otherwise an IEEE division (hipcc keeps fp32 division correctly
  // rounded by default).
  if constexpr ((R & (R - 1)) == 0) return acc * scale;
  else return acc / static_cast<float>(R);
}

__device__ __forceinline__ float finish_rt(float acc, int R, float scale, bool pow2) {
  return pow2 ? acc * scale : acc / static_cast<float>(R);
}

template <int R>
__device__ __forceinline__ v4f mean4(const v4f (&x)[R], float scale) {
  v4f a = x[0];
#pragma unroll
  for (int r = 1; r < R; ++r) {
    a.x = a.x + x[r].x;
    a.y = a.y + x[r].y;
    a.z = a.z + x[r].z;
    a.w = a.w + x[r].w;
  }
  a.x = finish<R>(a.x, scale);
  a.y = finish<R>(a.y, scale);
  a.z = finish<R>(a.z, scale);
  a.w = finish<R>(a.w, scale);
  return a;
}

// Device clock stamps of one launch: [0] start (first block), [1] end (last
// block to finish), [2] finished-block counter, reset by the last block.
__device__ __forceinline__ void stamp_begin(int64_t* stamp) {
  if (stamp != nullptr && blockIdx.x == 0 && threadIdx.x == 0) stamp[0] = static_cast<int64_t>(wall_clock64());
}

__device__ __forceinline__ void stamp_end(int64_t* stamp) {
  if (stamp == nullptr) return;
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const unsigned long long prev = atomicAdd(reinterpret_cast<unsigned long long*>(stamp + 2), 1ull);
    if (prev == gridDim.x - 1) {
      stamp[1] = static_cast<int64_t>(wall_clock64());
      stamp[2] = 0;
    }
  }
}

template <int R>
struct Unroll {
  static constexpr int value = R <= 2 ? 8 : (R <= 8 ? 4 : 2);
};

// ---------------------------------------------------------------------------
// fused gather + mean + copy-back, one wavefront per segment

// Which replicas contribute to variable `var` (bit r), from the R x P used
// flags; all replicas when there are no flags.
template <typename M>
__device__ __forceinline__ M used_mask(const uint8_t* used, int32_t var, int32_t P, int R) {
  if (used == nullptr) return R >= static_cast<int>(sizeof(M) * 8) ? ~M(0) : ((M(1) << R) - 1);
  M m = 0;
  for (int r = 0; r < R; ++r) m |= static_cast<M>(used[static_cast<int64_t>(r) * P + var] ? 1 : 0) << r;
  return m;
}

// Bucket views with used flags: a variable no replica used still has its
// bucket slices averaged (all zero-filled), so every replica's view becomes
// +0.0. Writes zeros to `len` elements at p.
__device__ __forceinline__ void zero_fill(float* p, int len, int lane, bool vec) {
  int tail = 0;
  if (vec) {
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    const int n4 = len >> 2;
    const __amdgpu_buffer_rsrc_t rp = seg_rsrc(p, n4 * 16);
    for (int i = lane; i < n4; i += 64) bst4(rp, 16 * i, zero);
    tail = n4 * 4;
  }
  for (int j = tail + lane; j < len; j += 64) G(p)[j] = 0.0f;
}

// MASKED = false compiles the used-flag paths out: at R = 8, 168 VGPRs instead
// of 254 VGPRs + 16 AGPRs, so up to three of its waves share a SIMD. Run beside
// a bf16 GEMM backward with no limit on workgroups per CU it hid 0.16 of the
// reduction against 0.09-0.11 for one workgroup per CU. The launcher uses it
// for launches without used flags when workgroups may share CUs
// (ddpb_set_workgroups_per_cu 0 or 2). At one workgroup per CU the general
// build streamed 0.4 % faster (BERT-large sync: 5,757 vs 5,734 GB/s, three
// runs each on one box, both builds with plain non-temporal stores) and is
// used instead.
template <int R, bool MASKED>
__global__ __launch_bounds__(kBlock) void fused_mean_kernel(const Segment* __restrict__ segs, int32_t nseg,
                                                            float* const* __restrict__ grads, int32_t P,
                                                            float scale, int32_t vec_ok,
                                                            const uint8_t* __restrict__ used, int32_t zero_unused,
                                                            int64_t* __restrict__ stamp) {
  constexpr int U = Unroll<R>::value;
  constexpr uint32_t kAll = (1u << R) - 1;
  stamp_begin(stamp);
  // One wavefront per segment; with a capped grid (fewer workgroups than
  // segments / 4) each wavefront strides over the remaining segments.
  for (int s = blockIdx.x * kWavesPerBlock + wave_id(); s < nseg; s += gridDim.x * kWavesPerBlock) {
    const Segment g = segs[s];
    const int len = static_cast<int>(g.len);
    float* p[R];
#pragma unroll
    for (int r = 0; r < R; ++r) p[r] = grads[static_cast<int64_t>(r) * P + g.var] + g.start;
    const int lane = lane_id();
    const uint32_t mask = MASKED ? used_mask<uint32_t>(used, g.var, P, R) : kAll;
    uintptr_t any = 0;                       // 16-byte alignment of every replica's pointer
#pragma unroll
    for (int r = 0; r < R; ++r) any |= reinterpret_cast<uintptr_t>(p[r]);
    if (MASKED && mask == 0) {               // no replica used it
      if (zero_unused) {                     // bucket views: the averaged zero slices
        const bool vz = vec_ok && (g.flags & kSegVecStart) && (any & 15) == 0;
#pragma unroll
        for (int r = 0; r < R; ++r) zero_fill(p[r], len, lane, vz);
      }
      continue;                              // copy modes: every gradient left untouched
    }
    if (MASKED && mask != kAll) {
      // Some replicas did not use this variable: their bucket slice is zero,
      // so they add +0.0 in their place of the fixed order (their gradients
      // are not read). The mask is the same for the whole wavefront.
      constexpr int UM = 2;
      int mtail = 0;
      if (vec_ok && (g.flags & kSegVecStart) && (any & 15) == 0) {
        const int n4 = len >> 2;
        const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
        __amdgpu_buffer_rsrc_t rr[R];
#pragma unroll
        for (int r = 0; r < R; ++r) rr[r] = seg_rsrc(p[r], n4 * 16);
        for (int i = lane; i < n4; i += 64 * UM) {
          v4f x[UM][R];
#pragma unroll
          for (int u = 0; u < UM; ++u)
#pragma unroll
            for (int r = 0; r < R; ++r)
              if (i + 64 * u < n4) x[u][r] = ((mask >> r) & 1u) ? bld4(rr[r], 16 * (i + 64 * u)) : zero;
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < UM; ++u) {
            if (i + 64 * u < n4) {
              const v4f m = mean4<R>(x[u], scale);
#pragma unroll
              for (int r = 0; r < R; ++r) bst4(rr[r], 16 * (i + 64 * u), m);
            }
          }
        }
        mtail = n4 * 4;
      }
      for (int j = mtail + lane; j < len; j += 64) {
        float x[R];
#pragma unroll
        for (int r = 0; r < R; ++r) x[r] = ((mask >> r) & 1u) ? G(p[r])[j] : 0.0f;
        float a = x[0];
#pragma unroll
        for (int r = 1; r < R; ++r) a = a + x[r];
        const float m = finish<R>(a, scale);
#pragma unroll
        for (int r = 0; r < R; ++r) G(p[r])[j] = m;
      }
      continue;
    }
    int tail = 0;
    if (vec_ok && (g.flags & kSegVecStart) && (any & 15) == 0) {
      const int n4 = len >> 2;
      // The general build goes through buffer resources (device-scope
      // stores); the compact build keeps global-pointer accesses with plain
      // non-temporal stores. Beside the bf16 backward with no per-CU limit the
      // compact build's buffer form made the step about 1 ms slower (MLP, 24
      // layers, R = 8: 31.92-32.11 against 30.98-31.06 ms with the global
      // form, on one box, whether its stores carried device scope or not).
      __amdgpu_buffer_rsrc_t rr[R];
#pragma unroll
      for (int r = 0; r < R; ++r) rr[r] = seg_rsrc(p[r], MASKED ? n4 * 16 : 0);
      // Every access of the unrolled group carries its own bound check. The
      // checked loads after the first group then issue one at a time under
      // exec masks instead of back to back; on gfx950 this paced request
      // stream moves 4-6 % more bytes per second than an unchecked body with
      // a remainder loop (measured on 8 x 1.34 GB, separate and shared
      // allocations). It also covers the partial last group.
      for (int i = lane; i < n4; i += 64 * U) {
        v4f x[U][R];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int r = 0; r < R; ++r)
            if (i + 64 * u < n4) x[u][r] = MASKED ? bld4(rr[r], 16 * (i + 64 * u)) : ld4s(p[r] + 4 * (i + 64 * u));
        // Keep all U*R loads in flight: the scheduler may not sink them
        // between the adds (it would otherwise trade bandwidth for registers).
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (i + 64 * u < n4) {
            const v4f m = mean4<R>(x[u], scale);
#pragma unroll
            for (int r = 0; r < R; ++r) {
              if constexpr (MASKED) bst4(rr[r], 16 * (i + 64 * u), m);
              else st4s(p[r] + 4 * (i + 64 * u), m);
            }
          }
        }
      }
      tail = n4 * 4;
    }
    for (int j = tail + lane; j < len; j += 64) {
      float x[R];
#pragma unroll
      for (int r = 0; r < R; ++r) x[r] = G(p[r])[j];
      float a = x[0];
#pragma unroll
      for (int r = 1; r < R; ++r) a = a + x[r];
      const float m = finish<R>(a, scale);
#pragma unroll
      for (int r = 0; r < R; ++r) G(p[r])[j] = m;
    }
  }
  stamp_end(stamp);
}

// Any R (up to 64), runtime replica count, same arithmetic order: the
// replicas are taken in chunks of kRtChunk whose loads all issue before the
// chunk's adds (in replica order), two 1 KiB groups per lane in flight.
constexpr int kRtChunk = 8;
constexpr int kRtU = 2;

__global__ __launch_bounds__(kBlock) void fused_mean_kernel_rt(const Segment* __restrict__ segs, int32_t nseg,
                                                               float* const* __restrict__ grads, int32_t P,
                                                               int32_t R, float scale, int32_t pow2,
                                                               int32_t vec_ok, const uint8_t* __restrict__ used,
                                                               int32_t zero_unused, int64_t* __restrict__ stamp) {
  stamp_begin(stamp);
  // One wavefront per segment; with a capped grid (fewer workgroups than
  // segments / 4) each wavefront strides over the remaining segments.
  for (int s = blockIdx.x * kWavesPerBlock + wave_id(); s < nseg; s += gridDim.x * kWavesPerBlock) {
    const Segment g = segs[s];
    const int len = static_cast<int>(g.len);
    const int lane = lane_id();
    const uint64_t mask = used_mask<uint64_t>(used, g.var, P, R);
    if (mask == 0) {                         // no replica used it: see fused_mean_kernel
      if (zero_unused)
        for (int r = 0; r < R; ++r) zero_fill(grads[static_cast<int64_t>(r) * P + g.var] + g.start, len, lane, false);
      continue;
    }
    int tail = 0;
    if (vec_ok && (g.flags & kSegVecStart)) {
      uintptr_t any = 0;                     // 16-byte alignment of every replica's pointer
      for (int r = 0; r < R; ++r) any |= reinterpret_cast<uintptr_t>(grads[static_cast<int64_t>(r) * P + g.var]);
      if (((any + static_cast<uintptr_t>(g.start) * 4) & 15) == 0) {
        const int n4 = len >> 2;
        for (int i = lane; i < n4; i += 64 * kRtU) {
          v4f a[kRtU];
          for (int r0 = 0; r0 < R; r0 += kRtChunk) {
            v4f x[kRtU][kRtChunk];
#pragma unroll
            for (int u = 0; u < kRtU; ++u)
#pragma unroll
              for (int q = 0; q < kRtChunk; ++q)
                if (r0 + q < R && i + 64 * u < n4)
                  x[u][q] = ((mask >> (r0 + q)) & 1u)   // +0.0 for a replica that did not use it
                                ? ld4s(grads[static_cast<int64_t>(r0 + q) * P + g.var] + g.start + 4 * (i + 64 * u))
                                : v4f{0.0f, 0.0f, 0.0f, 0.0f};
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < kRtU; ++u) {
              if (i + 64 * u < n4) {
#pragma unroll
                for (int q = 0; q < kRtChunk; ++q) {
                  if (r0 + q < R) {
                    if (r0 + q == 0) {
                      a[u] = x[u][q];
                    } else {
                      a[u].x = a[u].x + x[u][q].x;
                      a[u].y = a[u].y + x[u][q].y;
                      a[u].z = a[u].z + x[u][q].z;
                      a[u].w = a[u].w + x[u][q].w;
                    }
                  }
                }
              }
            }
          }
#pragma unroll
          for (int u = 0; u < kRtU; ++u) {
            if (i + 64 * u < n4) {
              v4f m;
              m.x = finish_rt(a[u].x, R, scale, pow2 != 0);
              m.y = finish_rt(a[u].y, R, scale, pow2 != 0);
              m.z = finish_rt(a[u].z, R, scale, pow2 != 0);
              m.w = finish_rt(a[u].w, R, scale, pow2 != 0);
              for (int r = 0; r < R; ++r)
                bst4(seg_rsrc(grads[static_cast<int64_t>(r) * P + g.var] + g.start, n4 * 16), 16 * (i + 64 * u), m);
            }
          }
        }
        tail = n4 * 4;
      }
    }
    // Scalar path: ragged tails and unaligned views (a replica that did not
    // use the variable holds +0.0 in its place of the order).
    for (int j = tail + lane; j < len; j += 64) {
      float a = (mask & 1u) ? G(grads[g.var])[g.start + j] : 0.0f;
      for (int r = 1; r < R; ++r)
        a = a + (((mask >> r) & 1u) ? G(grads[static_cast<int64_t>(r) * P + g.var])[g.start + j] : 0.0f);
      const float m = finish_rt(a, R, scale, pow2 != 0);
      for (int r = 0; r < R; ++r) G(grads[static_cast<int64_t>(r) * P + g.var])[g.start + j] = m;
    }
  }
  stamp_end(stamp);
}

// ---------------------------------------------------------------------------
// staged path

// Unroll of the staged kernels' copy loops (bound-checked groups, as in the
// fused kernel). Gradients are streamed non-temporally; the flat buckets use
// ordinary accesses so that a bucket packed by one kernel can still be in the
// Infinity Cache when the mean kernel reads it.
constexpr int kPackU = 8;
constexpr int kCopybackU = 4;

// R gradients -> R flat buckets (the narrowed views of [Li] "Gradient
// Bucketing": view.copy_(grad)).
__global__ __launch_bounds__(kBlock) void pack_kernel(const Segment* __restrict__ segs, int32_t nseg,
                                                      float* const* __restrict__ grads, int32_t P, int32_t R,
                                                      float* __restrict__ flat, int64_t flat_stride,
                                                      int64_t fbase, int32_t vec_ok,
                                                      const uint8_t* __restrict__ used,
                                                      int64_t* __restrict__ stamp) {
  stamp_begin(stamp);
  // One wavefront per segment; with a capped grid (fewer workgroups than
  // segments / 4) each wavefront strides over the remaining segments.
  for (int s = blockIdx.x * kWavesPerBlock + wave_id(); s < nseg; s += gridDim.x * kWavesPerBlock) {
    const Segment g = segs[s];
    const int len = static_cast<int>(g.len);
    const int lane = lane_id();
    const bool vec = vec_ok && (g.flags & kSegVecBoth) == kSegVecBoth;
    for (int r = 0; r < R; ++r) {
      const float* src = grads[static_cast<int64_t>(r) * P + g.var] + g.start;
      float* dst = flat + r * flat_stride + fbase + g.boff;
      if (used != nullptr && !used[static_cast<int64_t>(r) * P + g.var]) {
        for (int j = lane; j < len; j += 64) G(dst)[j] = 0.0f;   // unused here: zero slice
        continue;
      }
      int tail = 0;
      if (vec && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
        const int n4 = len >> 2;
        for (int i = lane; i < n4; i += 64 * kPackU) {
          v4f x[kPackU];
#pragma unroll
          for (int u = 0; u < kPackU; ++u)
            if (i + 64 * u < n4) x[u] = ld4s(src + 4 * (i + 64 * u));
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < kPackU; ++u)
            if (i + 64 * u < n4) st4(dst + 4 * (i + 64 * u), x[u]);
        }
        tail = n4 * 4;
      }
      for (int j = tail + lane; j < len; j += 64) G(dst)[j] = G(src)[j];
    }
  }
  stamp_end(stamp);
}

// R flat buckets -> averaged bucket; grid-stride over contiguous v4fs, kMeanU
// of them per thread in flight (bound-checked, as in the fused kernel).
constexpr int kMeanU = 4;

template <int R>
__global__ __launch_bounds__(kBlock) void mean_kernel(const float* __restrict__ flat, int64_t flat_stride,
                                                      int64_t fbase, int64_t n, float* __restrict__ avg,
                                                      float scale, int64_t* __restrict__ stamp) {
  stamp_begin(stamp);
  const float* src = flat + fbase;
  float* dst = avg + fbase;
  const int64_t n4 = n >> 2;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n4; i += kMeanU * stride) {
    v4f x[kMeanU][R];
#pragma unroll
    for (int u = 0; u < kMeanU; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (i + u * stride < n4) x[u][r] = ld4(src + r * flat_stride + 4 * (i + u * stride));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kMeanU; ++u)
      if (i + u * stride < n4) st4(dst + 4 * (i + u * stride), mean4<R>(x[u], scale));
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t j = n4 * 4 + threadIdx.x;
    float a = G(src)[j];
#pragma unroll
    for (int r = 1; r < R; ++r) a = a + G(src)[r * flat_stride + j];
    G(dst)[j] = finish<R>(a, scale);
  }
  stamp_end(stamp);
}

__global__ __launch_bounds__(kBlock) void mean_kernel_rt(const float* __restrict__ flat, int64_t flat_stride,
                                                         int64_t fbase, int64_t n, float* __restrict__ avg,
                                                         int32_t R, float scale, int32_t pow2,
                                                         int64_t* __restrict__ stamp) {
  stamp_begin(stamp);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t j = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; j < n; j += stride) {
    float a = G(flat)[fbase + j];
    for (int r = 1; r < R; ++r) a = a + G(flat)[r * flat_stride + fbase + j];
    G(avg)[fbase + j] = finish_rt(a, R, scale, pow2 != 0);
  }
  stamp_end(stamp);
}

// averaged bucket -> R gradients ([TP] "Internal Design": one batched copy per
// bucket back into the grad fields).
__global__ __launch_bounds__(kBlock) void copyback_kernel(const Segment* __restrict__ segs, int32_t nseg,
                                                          float* const* __restrict__ grads, int32_t P, int32_t R,
                                                          const float* __restrict__ avg, int64_t fbase,
                                                          int32_t vec_ok, const uint8_t* __restrict__ used,
                                                          int64_t* __restrict__ stamp) {
  stamp_begin(stamp);
  // One wavefront per segment; with a capped grid (fewer workgroups than
  // segments / 4) each wavefront strides over the remaining segments.
  for (int s = blockIdx.x * kWavesPerBlock + wave_id(); s < nseg; s += gridDim.x * kWavesPerBlock) {
    const Segment g = segs[s];
    if (used_mask<uint64_t>(used, g.var, P, R) == 0) continue;   // globally unused: untouched
    const int len = static_cast<int>(g.len);
    const int lane = lane_id();
    const float* src = avg + fbase + g.boff;
    uintptr_t any = 0;
    for (int r = 0; r < R; ++r)
      any |= reinterpret_cast<uintptr_t>(grads[static_cast<int64_t>(r) * P + g.var] + g.start);
    const bool vec = vec_ok && (g.flags & kSegVecBoth) == kSegVecBoth && (any & 15) == 0;
    int tail = 0;
    if (vec) {
      const int n4 = len >> 2;
      for (int i = lane; i < n4; i += 64 * kCopybackU) {
        v4f m[kCopybackU];
#pragma unroll
        for (int u = 0; u < kCopybackU; ++u)
          if (i + 64 * u < n4) m[u] = ld4(src + 4 * (i + 64 * u));
        __builtin_amdgcn_sched_barrier(0);
        for (int r = 0; r < R; ++r) {
          const __amdgpu_buffer_rsrc_t rd = seg_rsrc(grads[static_cast<int64_t>(r) * P + g.var] + g.start, n4 * 16);
#pragma unroll
          for (int u = 0; u < kCopybackU; ++u)
            if (i + 64 * u < n4) bst4(rd, 16 * (i + 64 * u), m[u]);
        }
      }
      tail = n4 * 4;
    }
    for (int j = tail + lane; j < len; j += 64) {
      const float m = G(src)[j];
      for (int r = 0; r < R; ++r) G(grads[static_cast<int64_t>(r) * P + g.var])[g.start + j] = m;
    }
  }
  stamp_end(stamp);
}

// ---------------------------------------------------------------------------
// no_sync accumulation ([Li] "Gradient Accumulation (no_sync)": .grad adds up
// across backward passes). One wavefront per (segment, replica).

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);   // exact widening
}

// Unroll of the accumulation loop and whether it bypasses the caches (each
// byte is touched once per micro-step; the accumulators of a large model do
// not stay cached from one micro-step to the next). The add stores with device
// scope as the reduction does (BERT-base shapes, R = 16, bf16: 2.712-2.714
// against 2.758-2.761 ms per micro-step, three interleaved runs each); the
// first micro-step, which only writes, and the synchronising step kept their
// plain non-temporal stores (device scope: first micro-step 1.712-1.713 against
// 1.695-1.698 ms, synchronising step no faster).
constexpr int kAccU = 8;
// Synchronising step (fused_acc_mean_kernel): replicas per chunk and float4
// groups per lane in flight. Every load of a chunk issues before its adds:
// 16 replicas x 2 groups = 32 accumulator and 32 step loads per lane.
constexpr int kAccMeanChunk = 16;
constexpr int kAccMeanU = 2;
constexpr bool kAccNT = true;

template <bool NT>
__device__ __forceinline__ v4f ld4x(const float* p) { if constexpr (NT) return ld4s(p); else return ld4(p); }
template <bool NT>
__device__ __forceinline__ void st4x(float* p, v4f v) { if constexpr (NT) st4s(p, v); else st4(p, v); }
template <bool NT>
__device__ __forceinline__ v2u ld2x(const uint16_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load((const gv2u*)p); else return *(const gv2u*)p;
}

template <bool BF16, bool FIRST>
__global__ __launch_bounds__(kBlock) void accumulate_kernel(const Segment* __restrict__ segs, int32_t nseg,
                                                            float* const* __restrict__ grads,
                                                            const void* const* __restrict__ steps, int32_t P,
                                                            int32_t R, int32_t vec_ok) {
  constexpr int U = kAccU;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave_id();
  if (w >= static_cast<int64_t>(nseg) * R) return;
  const int r = static_cast<int>(w / nseg);
  const Segment g = segs[w - static_cast<int64_t>(r) * nseg];
  const int len = static_cast<int>(g.len);
  const int64_t k = static_cast<int64_t>(r) * P + g.var;
  float* acc = grads[k] + g.start;
  const int lane = lane_id();
  if (steps[k] == nullptr) {                 // no gradient from this replica in this micro-step
    if (FIRST)
      for (int j = lane; j < len; j += 64) G(acc)[j] = 0.0f;
    return;
  }
  int tail = 0;
  // The unrolled groups check every access against the end, as in the fused
  // mean kernel (paced loads, no remainder loop).
  if (BF16) {
    const uint16_t* st = static_cast<const uint16_t*>(steps[k]) + g.start;
    if (vec_ok && (g.flags & kSegVecStart) && (reinterpret_cast<uintptr_t>(acc) & 15) == 0 &&
        (reinterpret_cast<uintptr_t>(st) & 7) == 0) {
      const int n4 = len >> 2;
      const __amdgpu_buffer_rsrc_t racc = seg_rsrc(acc, n4 * 16);
      for (int i = lane; i < n4; i += 64 * U) {
        v2u b[U];
        v4f a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (i + 64 * u < n4) {
            b[u] = ld2x<kAccNT>(st + 4 * (i + 64 * u));
            if (!FIRST) a[u] = ld4x<kAccNT>(acc + 4 * (i + 64 * u));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (i + 64 * u < n4) {
            v4f s4;
            s4.x = __uint_as_float(b[u].x << 16);
            s4.y = __uint_as_float(b[u].x & 0xffff0000u);
            s4.z = __uint_as_float(b[u].y << 16);
            s4.w = __uint_as_float(b[u].y & 0xffff0000u);
            if (!FIRST) {
              s4.x = a[u].x + s4.x;
              s4.y = a[u].y + s4.y;
              s4.z = a[u].z + s4.z;
              s4.w = a[u].w + s4.w;
            }
            if (FIRST) st4x<kAccNT>(acc + 4 * (i + 64 * u), s4);
            else bst4(racc, 16 * (i + 64 * u), s4);
          }
        }
      }
      tail = n4 * 4;
    }
    for (int j = tail + lane; j < len; j += 64) {
      const float s1 = bf16_to_f32(((const __attribute__((address_space(1))) uint16_t*)st)[j]);
      G(acc)[j] = FIRST ? s1 : G(acc)[j] + s1;
    }
  } else {
    const float* st = static_cast<const float*>(steps[k]) + g.start;
    if (vec_ok && (g.flags & kSegVecStart) &&
        ((reinterpret_cast<uintptr_t>(acc) | reinterpret_cast<uintptr_t>(st)) & 15) == 0) {
      const int n4 = len >> 2;
      const __amdgpu_buffer_rsrc_t racc = seg_rsrc(acc, n4 * 16);
      for (int i = lane; i < n4; i += 64 * U) {
        v4f b[U];
        v4f a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (i + 64 * u < n4) {
            b[u] = ld4x<kAccNT>(st + 4 * (i + 64 * u));
            if (!FIRST) a[u] = ld4x<kAccNT>(acc + 4 * (i + 64 * u));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (i + 64 * u < n4) {
            v4f s4 = b[u];
            if (!FIRST) {
              s4.x = a[u].x + s4.x;
              s4.y = a[u].y + s4.y;
              s4.z = a[u].z + s4.z;
              s4.w = a[u].w + s4.w;
            }
            if (FIRST) st4x<kAccNT>(acc + 4 * (i + 64 * u), s4);
            else bst4(racc, 16 * (i + 64 * u), s4);
          }
        }
      }
      tail = n4 * 4;
    }
    for (int j = tail + lane; j < len; j += 64) G(acc)[j] = FIRST ? G(st)[j] : G(acc)[j] + G(st)[j];
  }
}


// The synchronising micro-step fused into the reduction ([Li] "Gradient
// Accumulation (no_sync)": the last local backward accumulates into the
// gradients, then the buckets are averaged). Each replica's gradient enters
// the mean as accumulate_kernel would leave it -- float(step) on a first
// step, grad + float(step) otherwise, grad itself where the replica has no
// step (NULL; +0.0 on a first step) -- summed in replica order and divided
// once; the mean is written back. One HBM pass instead of an accumulation
// pass and a reduction pass. Replica count at run time, replicas in chunks of
// kAccMeanChunk.
// The loads and the arithmetic are separate so that a group issues every
// replica's loads before it consumes any: an add next to the loads (or a branch
// on a NULL step between them) makes the compiler wait for each replica's loads
// before issuing the next replica's, one round trip per replica.
template <bool BF16>
struct StepRaw {
  typedef v4f T;                             // fp32 step: four floats
};
template <>
struct StepRaw<true> {
  typedef v2u T;                             // bf16 step: four bf16 in two dwords
};

template <bool BF16>
__device__ __forceinline__ typename StepRaw<BF16>::T step_ld4(const void* step, int64_t e) {
  if constexpr (BF16) return __builtin_nontemporal_load((const gv2u*)(static_cast<const uint16_t*>(step) + e));
  else return ld4s(static_cast<const float*>(step) + e);
}

// What the accumulation would leave in one replica's gradient: float(step) on
// a first step, acc + float(step) otherwise; acc where the replica has no step
// (+0.0 on a first step). `raw` is read only when has_step.
template <bool BF16, bool FIRST>
__device__ __forceinline__ v4f acc_combine4(v4f acc, const typename StepRaw<BF16>::T& raw, bool has_step) {
  if (!has_step) {
    if (FIRST) return v4f{0.0f, 0.0f, 0.0f, 0.0f};
    return acc;
  }
  v4f s4;
  if constexpr (BF16) {
    s4.x = __uint_as_float(raw.x << 16);
    s4.y = __uint_as_float(raw.x & 0xffff0000u);
    s4.z = __uint_as_float(raw.y << 16);
    s4.w = __uint_as_float(raw.y & 0xffff0000u);
  } else {
    s4 = raw;
  }
  if (FIRST) return s4;
  acc.x = acc.x + s4.x;
  acc.y = acc.y + s4.y;
  acc.z = acc.z + s4.z;
  acc.w = acc.w + s4.w;
  return acc;
}

template <bool BF16, bool FIRST>
__device__ __forceinline__ float acc_step1(const float* acc, const void* step, int64_t e) {
  const float a = FIRST ? 0.0f : G(acc)[e];
  if (step == nullptr) return a;
  const float s1 = BF16 ? bf16_to_f32(((const __attribute__((address_space(1))) uint16_t*)step)[e])
                        : ((const gfloat*)step)[e];
  return FIRST ? s1 : a + s1;
}

template <bool BF16, bool FIRST>
__global__ __launch_bounds__(kBlock) void fused_acc_mean_kernel(const Segment* __restrict__ segs, int32_t nseg,
                                                                float* const* __restrict__ grads,
                                                                const void* const* __restrict__ steps, int32_t P,
                                                                int32_t R, float scale, int32_t pow2, int32_t vec_ok,
                                                                int64_t* __restrict__ stamp) {
  stamp_begin(stamp);
  // One wavefront per segment; with a capped grid (fewer workgroups than
  // segments / 4) each wavefront strides over the remaining segments.
  for (int s = blockIdx.x * kWavesPerBlock + wave_id(); s < nseg; s += gridDim.x * kWavesPerBlock) {
    const Segment g = segs[s];
    const int len = static_cast<int>(g.len);
    const int lane = lane_id();
    int tail = 0;
    if (vec_ok && (g.flags & kSegVecStart)) {
      uintptr_t any = 0, anys = 0;           // alignment of every gradient (16 B) and step (8 / 16 B)
      for (int r = 0; r < R; ++r) {
        const int64_t k = static_cast<int64_t>(r) * P + g.var;
        any |= reinterpret_cast<uintptr_t>(grads[k] + g.start);
        if (steps[k] != nullptr)
          anys |= reinterpret_cast<uintptr_t>(steps[k]) + static_cast<uintptr_t>(g.start) * (BF16 ? 2 : 4);
      }
      if ((any & 15) == 0 && (anys & (BF16 ? 7 : 15)) == 0) {
        const int n4 = len >> 2;
        for (int i = lane; i < n4; i += 64 * kAccMeanU) {
          v4f a[kAccMeanU];
          for (int r0 = 0; r0 < R; r0 += kAccMeanChunk) {
            const float* ap[kAccMeanChunk];
            const void* sp[kAccMeanChunk];
#pragma unroll
            for (int q = 0; q < kAccMeanChunk; ++q) {
              const int64_t k = static_cast<int64_t>(r0 + q < R ? r0 + q : 0) * P + g.var;
              ap[q] = grads[k];
              sp[q] = steps[k];
            }
            v4f x[kAccMeanU][kAccMeanChunk];
            typename StepRaw<BF16>::T y[kAccMeanU][kAccMeanChunk];
            // Every accumulator load of the group first, then every step load:
            // 7.5 % faster than alternating the two per replica (BERT-base,
            // R = 16, bf16: 3.01-3.03 against 3.26-3.28 ms).
#pragma unroll
            for (int u = 0; u < kAccMeanU; ++u)
#pragma unroll
              for (int q = 0; q < kAccMeanChunk; ++q)
                if (r0 + q < R && i + 64 * u < n4)
                  x[u][q] = FIRST ? v4f{0.0f, 0.0f, 0.0f, 0.0f} : ld4s(ap[q] + g.start + 4 * (i + 64 * u));
#pragma unroll
            for (int u = 0; u < kAccMeanU; ++u)
#pragma unroll
              for (int q = 0; q < kAccMeanChunk; ++q)
                if (r0 + q < R && i + 64 * u < n4 && sp[q] != nullptr)   // else never read
                  y[u][q] = step_ld4<BF16>(sp[q], g.start + 4 * (i + 64 * u));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < kAccMeanU; ++u) {
              if (i + 64 * u < n4) {
#pragma unroll
                for (int q = 0; q < kAccMeanChunk; ++q) {
                  if (r0 + q < R) {
                    const v4f v = acc_combine4<BF16, FIRST>(x[u][q], y[u][q], sp[q] != nullptr);
                    if (r0 + q == 0) {
                      a[u] = v;
                    } else {
                      a[u].x = a[u].x + v.x;
                      a[u].y = a[u].y + v.y;
                      a[u].z = a[u].z + v.z;
                      a[u].w = a[u].w + v.w;
                    }
                  }
                }
              }
            }
          }
#pragma unroll
          for (int u = 0; u < kAccMeanU; ++u) {
            if (i + 64 * u < n4) {
              v4f m;
              m.x = finish_rt(a[u].x, R, scale, pow2 != 0);
              m.y = finish_rt(a[u].y, R, scale, pow2 != 0);
              m.z = finish_rt(a[u].z, R, scale, pow2 != 0);
              m.w = finish_rt(a[u].w, R, scale, pow2 != 0);
              for (int r = 0; r < R; ++r)
                st4s(grads[static_cast<int64_t>(r) * P + g.var] + g.start + 4 * (i + 64 * u), m);
            }
          }
        }
        tail = n4 * 4;
      }
    }
    // scalar path: ragged tails and unaligned pointers
    for (int j = tail + lane; j < len; j += 64) {
      float a = acc_step1<BF16, FIRST>(grads[g.var], steps[g.var], g.start + j);
      for (int r = 1; r < R; ++r) {
        const int64_t k = static_cast<int64_t>(r) * P + g.var;
        a = a + acc_step1<BF16, FIRST>(grads[k], steps[k], g.start + j);
      }
      const float m = finish_rt(a, R, scale, pow2 != 0);
      for (int r = 0; r < R; ++r) G(grads[static_cast<int64_t>(r) * P + g.var])[g.start + j] = m;
    }
  }
  stamp_end(stamp);
}

// ---------------------------------------------------------------------------
// launcher

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// A host-side roctx range over one launcher call (bindings made with
// DDPB_BIND_ROCTX), so that a marker trace shows when the host issued what.
class HostRange {
 public:
  HostRange(bool on, const char* what) : on_(on) {
    if (on_) roctxRangePushA(what);
  }
  ~HostRange() {
    if (on_) roctxRangePop();
  }
  HostRange(const HostRange&) = delete;
  HostRange& operator=(const HostRange&) = delete;

 private:
  bool on_;
};

// Whether work enqueued on `s` now is being recorded into a graph rather than
// run. A replayed graph repeats the recorded device work only, so anything
// that reads host memory at run time (a pinned-staging upload) or whose
// result the host reads back (launch-timing events) must not be recorded.
int capturing(hipStream_t s, bool* yes, std::string* err) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  HIP_OK(hipStreamIsCapturing(s, &st), "hipStreamIsCapturing");
  *yes = (st != hipStreamCaptureStatusNone);
  return kOk;
}

class HipLauncher final : public Launcher {
 public:
  ~HipLauncher() override { release(); }

  int bind(const Plan& plan, const BindArgs& a, std::string* err) override {
    const bool held_static = static_;
    release();
    if (a.no_alloc) return bind_static(plan, a, held_static, err);
    plan_ = &plan;
    R_ = plan.R;
    P_ = plan.P;
    mode_ = a.mode;
    flags_ = a.flags;
    compute_ = static_cast<hipStream_t>(a.compute_stream);
    side_.clear();
    for (void* s : a.side_streams) side_.push_back(static_cast<hipStream_t>(s));
    side_used_.assign(side_.size(), 0);
    pow2_ = (R_ & (R_ - 1)) == 0;
    scale_ = 1.0f / static_cast<float>(R_);
    vec_ok_ = 1;                // 128-bit paths are chosen per segment from pointer alignment
    flat_ = nullptr;
    avg_ = nullptr;
    if (mode_ == 1) {
      if (!aligned(a.workspace, 256)) {
        *err = "bind: workspace must be 256-byte aligned";
        return kErrArg;
      }
      flat_ = static_cast<float*>(a.workspace);
      avg_ = flat_ + static_cast<int64_t>(R_) * plan.flat_elems;
    }
    HIP_OK(hipGetDevice(&device_), "hipGetDevice");

    const size_t nptr = static_cast<size_t>(R_) * P_;
    const size_t B = static_cast<size_t>(plan.B());
    HIP_OK(hipMalloc(&d_grads_, std::max<size_t>(nptr, 1) * sizeof(float*)), "hipMalloc(pointer table)");
    HIP_OK(hipMalloc(&d_segs_, std::max<size_t>(plan.segs.size(), 1) * sizeof(Segment)), "hipMalloc(segments)");
    HIP_OK(hipMalloc(&d_stamps_, std::max<size_t>(B, 1) * 4 * sizeof(int64_t)), "hipMalloc(stamps)");
    HIP_OK(hipMalloc(&d_steps_, std::max<size_t>(nptr, 1) * kStepSlots * sizeof(void*)), "hipMalloc(step tables)");
    HIP_OK(hipHostMalloc(&h_steps_, std::max<size_t>(nptr, 1) * kStepSlots * sizeof(void*), hipHostMallocDefault),
           "hipHostMalloc(step staging)");
    HIP_OK(hipMalloc(&d_used_, std::max<size_t>(nptr, 1)), "hipMalloc(used flags)");
    HIP_OK(hipMalloc(&d_sync_steps_, std::max<size_t>(nptr, 1) * sizeof(void*)), "hipMalloc(sync step table)");
    HIP_OK(hipHostMalloc(&h_sync_steps_, std::max<size_t>(nptr, 1) * sizeof(void*), hipHostMallocDefault),
           "hipHostMalloc(sync step staging)");
    HIP_OK(hipEventCreateWithFlags(&ev_sync_steps_, hipEventDisableTiming), "hipEventCreate");
    sync_steps_recorded_ = false;
    sync_step_active_ = false;
    HIP_OK(hipHostMalloc(&h_used_, std::max<size_t>(nptr, 1), hipHostMallocDefault), "hipHostMalloc(used staging)");
    HIP_OK(hipEventCreateWithFlags(&ev_used_, hipEventDisableTiming), "hipEventCreate");
    used_recorded_ = false;
    used_active_ = false;
    if (nptr)
      HIP_OK(hipMemcpyAsync(d_grads_, a.grad_ptrs.data(), nptr * sizeof(float*), hipMemcpyHostToDevice, compute_),
             "upload pointer table");
    if (!plan.segs.empty())
      HIP_OK(hipMemcpyAsync(d_segs_, plan.segs.data(), plan.segs.size() * sizeof(Segment), hipMemcpyHostToDevice,
                            compute_),
             "upload segment table");
    HIP_OK(hipMemsetAsync(d_stamps_, 0, std::max<size_t>(B, 1) * 4 * sizeof(int64_t), compute_), "clear stamps");
    if (mode_ == kModeBucketView) {
      for (void* p : a.view_bases)
        if (!aligned(p, 256)) {
          *err = "bind_bucket_views: every replica storage must be 256-byte aligned";
          return kErrArg;
        }
      HIP_OK(hipMalloc(&d_view_bases_, std::max<size_t>(R_, 1) * sizeof(float*)), "hipMalloc(view bases)");
      HIP_OK(hipMalloc(&d_view_segs_, std::max<size_t>(plan.view_segs.size(), 1) * sizeof(Segment)),
             "hipMalloc(view segments)");
      HIP_OK(hipMemcpyAsync(d_view_bases_, a.view_bases.data(), R_ * sizeof(float*), hipMemcpyHostToDevice, compute_),
             "upload view bases");
      if (!plan.view_segs.empty())
        HIP_OK(hipMemcpyAsync(d_view_segs_, plan.view_segs.data(), plan.view_segs.size() * sizeof(Segment),
                              hipMemcpyHostToDevice, compute_),
               "upload view segments");
    }
    HIP_OK(hipStreamSynchronize(compute_), "bind: synchronize");

    ev_ready_.assign(B, nullptr);
    for (auto& e : ev_ready_) HIP_OK(hipEventCreateWithFlags(&e, hipEventDisableTiming), "hipEventCreate");
    ev_done_.assign(side_.size(), nullptr);
    for (auto& e : ev_done_) HIP_OK(hipEventCreateWithFlags(&e, hipEventDisableTiming), "hipEventCreate");
    ev_tail_.assign(side_.size(), nullptr);
    tail_evt_.assign(side_.size(), nullptr);
    // Join events carried by the last kernels (with the system-scope fence,
    // as the markers they replace).
    for (auto& e : ev_tail_) HIP_OK(hipEventCreateWithFlags(&e, hipEventDisableTiming), "hipEventCreate");
    ev_slot_.assign(kStepSlots, nullptr);
    for (auto& e : ev_slot_) HIP_OK(hipEventCreateWithFlags(&e, hipEventDisableTiming), "hipEventCreate");
    slot_valid_.assign(kStepSlots, 0);
    slot_recorded_.assign(kStepSlots, 0);
    next_slot_ = 0;
    if (flags_ & 2) {
      ev_t0_.assign(B * kTimeRing, nullptr);
      ev_t1_.assign(B * kTimeRing, nullptr);
      // Timing only: no system-scope fence when these complete, which would
      // write back and invalidate caches between consecutive bucket kernels
      // (measured: the timed sync lost 1.5 % with default events, 0.8 % without
      // the fence). The end events of each side stream's last bucket keep the
      // fence: finalize's join waits on them, and what follows on the compute
      // stream may read the gradients through a copy engine.
      for (auto& e : ev_t0_) HIP_OK(hipEventCreateWithFlags(&e, hipEventDisableSystemFence), "hipEventCreate");
      for (size_t i = 0; i < ev_t1_.size(); ++i) {
        const bool tail = i % B + side_.size() >= B;
        HIP_OK(hipEventCreateWithFlags(&ev_t1_[i], tail ? hipEventDefault : hipEventDisableSystemFence),
               "hipEventCreate");
      }
    }
    // DDPB_BIND_OVERLAP: reduction workgroups may share CUs (with each other
    // and with the backward's kernels).
    if (flags_ & 8) wg_per_cu_ = 0;
    return update_lds_reserve(err);
  }

  int launch(int32_t first, int32_t last, int64_t iteration, std::string* err) override {
    if (static_ && !owns_scratch()) {
      *err = "launch: another handle's ddpb_bind_static has taken over this device's static tables; bind again";
      return kErrState;
    }
    char what[48] = "";
    if (flags_ & 4) std::snprintf(what, sizeof(what), "ddpb launch %d-%d", first, last);
    const HostRange range((flags_ & 4) != 0, what);
    const size_t ring = static_cast<size_t>(iteration % kTimeRing) * plan_->B();
    if (flags_ & 2) {
      bool cap = false;
      if (const int rc = capturing(compute_, &cap, err); rc != kOk) return rc;
      if (cap) {
        *err = "launch timing cannot be captured into a graph; bind without DDPB_BIND_TIME_LAUNCHES";
        return kErrState;
      }
    }
    // A bucket whose stream is the compute stream itself is ordered after the
    // gradients by the stream alone: no ready event, no wait, nothing to join.
    // A plan of one bucket always reduces on the compute stream: its bucket
    // launches only once the last gradient is ready, so a side stream could
    // overlap nothing and would add a fork and a join (nn.Linear(10,10), R = 2,
    // host-synchronised syncs: 15.6 against 48.1-48.5 us). With more buckets
    // the last one stays on its side stream (on the compute stream ResNet-50
    // shapes synced 4 % slower).
    const size_t ns = side_.size();
    const size_t nb = static_cast<size_t>(plan_->B());
    auto stream_of = [&](int32_t b) -> hipStream_t {
      return nb == 1 ? compute_ : side_[static_cast<size_t>(b) % ns];
    };
    bool fork = false;
    for (int32_t b = first; b <= last && !fork; ++b) fork = stream_of(b) != compute_;
    if (fork) HIP_OK(hipEventRecord(ev_ready_[first], compute_), "hipEventRecord(ready)");
    uint32_t waited = 0;
    // The last bucket of the iteration on each side stream carries the event
    // that finalize's join waits on as its kernel's completion event, so the
    // join needs no marker behind it on the side stream (one queue hop fewer
    // between a sync's last kernel and the compute stream: ResNet-50 shapes,
    // R = 8, 0.329 against 0.335 ms per sync). Not under stream capture, where
    // the join records its marker as before.
    auto is_tail = [&](int32_t b) { return stream_of(b) != compute_ && static_cast<size_t>(b) + ns >= nb; };
    bool tails = false;
    for (int32_t b = first; b <= last && !tails; ++b) tails = is_tail(b);
    if (tails) {
      bool cap = false;
      if (const int rc = capturing(compute_, &cap, err); rc != kOk) return rc;
      tails = !cap;
    }
    for (int32_t b = first; b <= last; ++b) {
      const size_t si = static_cast<size_t>(b) % side_.size();
      hipStream_t s = stream_of(b);
      if (s != compute_) {
        if (!(waited & (1u << si))) {
          HIP_OK(hipStreamWaitEvent(s, ev_ready_[first], 0), "hipStreamWaitEvent(ready)");
          waited |= 1u << si;
        }
        side_used_[si] = 1;
      }
      // Timing events ride on the kernel dispatches themselves (start of the
      // bucket's first kernel, end of its last), not on separate markers.
      hipEvent_t t0 = (flags_ & 2) ? ev_t0_[ring + b] : nullptr;
      hipEvent_t t1 = (flags_ & 2) ? ev_t1_[ring + b] : nullptr;
      const bool tail = tails && is_tail(b);
      if (tail && t1 == nullptr) t1 = ev_tail_[si];
      const int rc = enqueue_bucket(b, s, t0, t1, err);
      if (rc != kOk) return rc;
      if (tail) tail_evt_[si] = t1;          // completes with the stream's last kernel
    }
    return kOk;
  }

  int join(std::string* err) override {
    const HostRange range((flags_ & 4) != 0, "ddpb finalize join");
    for (size_t i = 0; i < side_.size(); ++i) {
      if (!side_used_[i]) continue;
      if (tail_evt_[i] != nullptr) {         // the stream's last bucket signals it
        HIP_OK(hipStreamWaitEvent(compute_, tail_evt_[i], 0), "hipStreamWaitEvent(tail)");
        tail_evt_[i] = nullptr;
      } else {                               // incomplete iteration, or captured
        HIP_OK(hipEventRecord(ev_done_[i], side_[i]), "hipEventRecord(done)");
        HIP_OK(hipStreamWaitEvent(compute_, ev_done_[i], 0), "hipStreamWaitEvent(done)");
      }
      side_used_[i] = 0;
    }
    return kOk;
  }

  int accumulate(void* const* step_ptrs, int32_t step_dtype, bool first, std::string* err) override {
    const HostRange range((flags_ & 4) != 0, "ddpb no_sync_accumulate");
    if (static_) {
      *err = "no_sync_accumulate: not available on a binding made by ddpb_bind_static";
      return kErrState;
    }
    const size_t nptr = static_cast<size_t>(R_) * P_;
    if (plan_->segs.empty()) return kOk;
    bool cap = false;
    if (const int rc = capturing(compute_, &cap, err); rc != kOk) return rc;
    if (cap) {                     // the step table comes from host staging that later calls reuse
      *err = "no_sync_accumulate cannot be captured into a graph";
      return kErrState;
    }
    const int vec = vec_ok_;       // alignment is checked per segment in the kernel
    // Step pointer tables go through a small ring of device slots; a table
    // seen recently is reused without another upload.
    int slot = -1;
    for (int k = 0; k < kStepSlots; ++k)
      if (slot_valid_[k] && std::memcmp(h_steps_ + k * nptr, step_ptrs, nptr * sizeof(void*)) == 0) slot = k;
    if (slot < 0) {
      slot = next_slot_;
      next_slot_ = (next_slot_ + 1) % kStepSlots;
      if (slot_recorded_[slot]) HIP_OK(hipEventSynchronize(ev_slot_[slot]), "hipEventSynchronize(slot)");
      std::memcpy(h_steps_ + slot * nptr, step_ptrs, nptr * sizeof(void*));
      HIP_OK(hipMemcpyAsync(d_steps_ + slot * nptr, h_steps_ + slot * nptr, nptr * sizeof(void*),
                            hipMemcpyHostToDevice, compute_),
             "upload step table");
      HIP_OK(hipEventRecord(ev_slot_[slot], compute_), "hipEventRecord(slot)");
      slot_recorded_[slot] = 1;
      slot_valid_[slot] = 1;
    }
    const int32_t nseg = static_cast<int32_t>(plan_->segs.size());
    const int64_t waves = static_cast<int64_t>(nseg) * R_;
    const dim3 grid(static_cast<unsigned>((waves + kWavesPerBlock - 1) / kWavesPerBlock));
    const void* const* tab = d_steps_ + slot * nptr;
    if (step_dtype == 1) {
      if (first)
        hipLaunchKernelGGL((accumulate_kernel<true, true>), grid, dim3(kBlock), lds_one_per_cu_, compute_, d_segs_,
                           nseg, d_grads_, tab, P_, R_, vec);
      else
        hipLaunchKernelGGL((accumulate_kernel<true, false>), grid, dim3(kBlock), lds_one_per_cu_, compute_, d_segs_,
                           nseg, d_grads_, tab, P_, R_, vec);
    } else {
      if (first)
        hipLaunchKernelGGL((accumulate_kernel<false, true>), grid, dim3(kBlock), lds_one_per_cu_, compute_, d_segs_,
                           nseg, d_grads_, tab, P_, R_, vec);
      else
        hipLaunchKernelGGL((accumulate_kernel<false, false>), grid, dim3(kBlock), lds_one_per_cu_, compute_, d_segs_,
                           nseg, d_grads_, tab, P_, R_, vec);
    }
    HIP_OK(hipGetLastError(), "launch accumulate_kernel");
    return kOk;
  }

  int read_stamps(const std::vector<LaunchRecord>& log, std::vector<int64_t>* t0, std::vector<int64_t>* t1,
                  std::string* err) override {
    const size_t B = static_cast<size_t>(plan_->B());
    std::vector<int64_t> h(std::max<size_t>(B, 1) * 4, 0);
    if (d_stamps_ != nullptr)        // (a static binding keeps no stamps)
      HIP_OK(hipMemcpy(h.data(), d_stamps_, h.size() * sizeof(int64_t), hipMemcpyDeviceToHost), "read stamps");
    t0->resize(log.size());
    t1->resize(log.size());
    for (size_t i = 0; i < log.size(); ++i) {
      (*t0)[i] = h[static_cast<size_t>(log[i].bucket) * 4 + 0];
      (*t1)[i] = h[static_cast<size_t>(log[i].bucket) * 4 + 1];
    }
    return kOk;
  }

  int read_times(int64_t iteration, const std::vector<LaunchRecord>& log, std::vector<float>* start_ms,
                 std::vector<float>* ms, std::string* err) override {
    if (!(flags_ & 2)) {
      *err = "launch timing was not enabled at bind";
      return kErrState;
    }
    const size_t ring = static_cast<size_t>(iteration % kTimeRing) * plan_->B();
    ms->resize(log.size());
    start_ms->resize(log.size());
    if (log.empty()) return kOk;
    const hipEvent_t ref = ev_t0_[ring + static_cast<size_t>(log[0].bucket)];
    for (size_t i = 0; i < log.size(); ++i) {
      const size_t b = ring + static_cast<size_t>(log[i].bucket);
      HIP_OK(hipEventSynchronize(ev_t1_[b]), "hipEventSynchronize(t1)");
      HIP_OK(hipEventElapsedTime(&(*ms)[i], ev_t0_[b], ev_t1_[b]), "hipEventElapsedTime");
      HIP_OK(hipEventElapsedTime(&(*start_ms)[i], ref, ev_t0_[b]), "hipEventElapsedTime");
    }
    return kOk;
  }

  void set_max_blocks(int32_t n) override { max_blocks_ = n; }

  int set_workgroups_per_cu(int32_t n, std::string* err) override {
    wg_per_cu_ = n;
    return update_lds_reserve(err);
  }

  int set_used(const uint8_t* used, const uint8_t* global, std::string* err) override {
    (void)global;                  // the kernels derive it from the per-replica flags
    if (used == nullptr) {
      used_active_ = false;
      return kOk;
    }
    if (static_) {
      *err = "used flags are not available on a binding made by ddpb_bind_static";
      return kErrState;
    }
    const size_t n = static_cast<size_t>(R_) * P_;
    if (n == 0) return kOk;
    bool cap = false;
    if (const int rc = capturing(compute_, &cap, err); rc != kOk) return rc;
    if (cap) {                     // the flags come from host staging that later calls reuse
      *err = "an iteration with used flags (ddpb_set_local_used) cannot be captured into a graph";
      return kErrState;
    }
    // The staging buffer may still feed the previous upload.
    if (used_recorded_) HIP_OK(hipEventSynchronize(ev_used_), "hipEventSynchronize(used)");
    std::memcpy(h_used_, used, n);
    HIP_OK(hipMemcpyAsync(d_used_, h_used_, n, hipMemcpyHostToDevice, compute_), "upload used flags");
    HIP_OK(hipEventRecord(ev_used_, compute_), "hipEventRecord(used)");
    used_recorded_ = true;
    used_active_ = true;
    return kOk;
  }

  int set_sync_step(void* const* step_ptrs, int32_t step_dtype, bool first, std::string* err) override {
    if (step_ptrs == nullptr) {
      sync_step_active_ = false;
      return kOk;
    }
    if (static_) {
      *err = "set_sync_step: not available on a binding made by ddpb_bind_static";
      return kErrState;
    }
    const HostRange range((flags_ & 4) != 0, "ddpb set_sync_step");
    const size_t n = static_cast<size_t>(R_) * P_;
    bool cap = false;
    if (const int rc = capturing(compute_, &cap, err); rc != kOk) return rc;
    if (cap) {                     // the table comes from host staging that later calls reuse
      *err = "ddpb_set_sync_step cannot be captured into a graph";
      return kErrState;
    }
    // The staging buffer may still feed the previous upload.
    if (sync_steps_recorded_) HIP_OK(hipEventSynchronize(ev_sync_steps_), "hipEventSynchronize(sync step)");
    std::memcpy(h_sync_steps_, step_ptrs, n * sizeof(void*));
    if (n)
      HIP_OK(hipMemcpyAsync(d_sync_steps_, h_sync_steps_, n * sizeof(void*), hipMemcpyHostToDevice, compute_),
             "upload sync step table");
    HIP_OK(hipEventRecord(ev_sync_steps_, compute_), "hipEventRecord(sync step)");
    sync_steps_recorded_ = true;
    sync_step_active_ = true;
    sync_step_bf16_ = (step_dtype == 1);
    sync_step_first_ = first;
    return kOk;
  }

  int clock_hz(int64_t* hz, std::string* err) override {
    int dev = 0, khz = 0;
    HIP_OK(hipGetDevice(&dev), "hipGetDevice");
    HIP_OK(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev), "wall clock rate");
    *hz = static_cast<int64_t>(khz) * 1000;
    return kOk;
  }

 private:
  // Allocation-free binding: the pointer and segment tables (and the staged
  // mode's flat buckets) are placed in this device's copy of `scratch`; the
  // reductions run on the compute stream, so no event is needed either.
  // Calls no hipMalloc, hipHostMalloc or hipEventCreate.
  int bind_static(const Plan& plan, const BindArgs& a, bool held_static, std::string* err) {
    plan_ = &plan;
    R_ = plan.R;
    P_ = plan.P;
    mode_ = a.mode;
    flags_ = 0;
    compute_ = static_cast<hipStream_t>(a.compute_stream);
    side_.assign(1, compute_);
    side_used_.assign(1, 0);
    tail_evt_.assign(1, nullptr);
    pow2_ = (R_ & (R_ - 1)) == 0;
    scale_ = 1.0f / static_cast<float>(R_);
    vec_ok_ = 1;
    flat_ = nullptr;
    avg_ = nullptr;
    HIP_OK(hipGetDevice(&device_), "hipGetDevice");
    char* base = nullptr;
    if (const int rc = static_scratch_base(device_, &base, err); rc != kOk) return rc;
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    const int64_t nptr = static_cast<int64_t>(R_) * P_;
    const int64_t off_segs = up(nptr * static_cast<int64_t>(sizeof(float*)));
    const int64_t off_flat = off_segs + up(static_cast<int64_t>(plan.segs.size() * sizeof(Segment)));
    const int64_t need = off_flat + (mode_ == kModeStaged ? workspace_bytes(plan, kModeStaged) : 0);
    if (need > kStaticScratchBytes) {
      *err = "bind_static: this model needs " + std::to_string(need) + " bytes of device tables" +
             (mode_ == kModeStaged ? " and flat buckets" : "") + ", the static array holds " +
             std::to_string(kStaticScratchBytes) + "; use ddpb_bind";
      plan_ = nullptr;
      return kErrArg;
    }
    const void* prev = nullptr;
    {
      std::lock_guard<std::mutex> lock(g_scratch_mu);
      prev = g_scratch_owner[device_];
      g_scratch_owner[device_] = this;
    }
    static_ = true;
    // The previous holder's reductions (another handle's, or this handle's
    // own earlier static binding, perhaps on another stream) may still read
    // the tables: let the device drain before they are overwritten.
    if ((prev != nullptr && prev != this) || held_static)
      HIP_OK(hipDeviceSynchronize(), "bind_static: synchronize");
    d_grads_ = reinterpret_cast<float**>(base);
    d_segs_ = reinterpret_cast<Segment*>(base + off_segs);
    if (mode_ == kModeStaged) {
      flat_ = reinterpret_cast<float*>(base + off_flat);
      avg_ = flat_ + static_cast<int64_t>(R_) * plan.flat_elems;
    }
    // Every byte the kernels read is written here (tables) or by the pack
    // kernel before the mean kernel reads it (flat buckets): nothing has to
    // start at zero.
    if (nptr)
      HIP_OK(hipMemcpyAsync(d_grads_, a.grad_ptrs.data(), nptr * sizeof(float*), hipMemcpyHostToDevice, compute_),
             "upload pointer table");
    if (!plan.segs.empty())
      HIP_OK(hipMemcpyAsync(d_segs_, plan.segs.data(), plan.segs.size() * sizeof(Segment), hipMemcpyHostToDevice,
                            compute_),
             "upload segment table");
    HIP_OK(hipStreamSynchronize(compute_), "bind_static: synchronize");
    return update_lds_reserve(err);
  }

  bool owns_scratch() const {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    return g_scratch_owner[device_] == this;
  }

  int enqueue_bucket(int32_t b, hipStream_t s, hipEvent_t t0, hipEvent_t t1, std::string* err) {
    // Bucket-view mode runs the same fused kernel over the bucket's flat range
    // of each replica's storage (one pseudo-variable per replica). With used
    // flags it walks the per-variable segments over the views instead, so
    // that unused replicas' slices count as zeros without being read and
    // variables no replica used end as zeros.
    const bool view = (mode_ == kModeBucketView) && !used_active_;
    const int32_t zero_unused = (mode_ == kModeBucketView && used_active_) ? 1 : 0;
    const std::vector<int32_t>& first = view ? plan_->view_seg_first : plan_->seg_first;
    const int32_t s0 = first[b];
    const int32_t nseg = first[b + 1] - s0;
    if (nseg == 0) {                          // bucket of empty tensors: nothing to move
      if (t0) HIP_OK(hipEventRecord(t0, s), "hipEventRecord(t0)");
      if (t1) HIP_OK(hipEventRecord(t1, s), "hipEventRecord(t1)");
      return kOk;
    }
    if (sync_step_active_) {
      // the synchronising micro-step: per-variable segments, steps per variable
      const int32_t v0 = plan_->seg_first[b];
      const int32_t vn = plan_->seg_first[b + 1] - v0;
      int64_t vblocks = (vn + kWavesPerBlock - 1) / kWavesPerBlock;
      if (max_blocks_ > 0) vblocks = std::min<int64_t>(vblocks, max_blocks_);
      const dim3 vgrid(static_cast<unsigned>(vblocks));
      const void* const* steps = d_sync_steps_;
      if ((mode_ == kModeFused || mode_ == kModeBucketView) && !used_active_) {
        const int32_t p2 = pow2_ ? 1 : 0;
        int64_t* st = (flags_ & 1) ? d_stamps_ + static_cast<int64_t>(b) * 4 : nullptr;
        // One workgroup per CU, as for the other streaming kernels (BERT-base,
        // R = 16, bf16: 3.27-3.29 ms per synchronising step against
        // 3.33-3.35 with no limit).
#define DDPB_ACC_MEAN(BF, FI)                                                                                   \
  hipExtLaunchKernelGGL((fused_acc_mean_kernel<BF, FI>), vgrid, dim3(kBlock), lds_one_per_cu_, s, t0, t1, 0,    \
                        d_segs_ + v0, vn, d_grads_, steps, P_, R_, scale_, p2, vec_ok_, st)
        if (sync_step_bf16_) {
          if (sync_step_first_) DDPB_ACC_MEAN(true, true); else DDPB_ACC_MEAN(true, false);
        } else {
          if (sync_step_first_) DDPB_ACC_MEAN(false, true); else DDPB_ACC_MEAN(false, false);
        }
#undef DDPB_ACC_MEAN
        HIP_OK(hipGetLastError(), "launch fused_acc_mean_kernel");
        return kOk;
      }
      // staged mode or used flags: accumulate the bucket's variables first,
      // on this side stream, then reduce as usual
      const dim3 agrid(static_cast<unsigned>((static_cast<int64_t>(vn) * R_ + kWavesPerBlock - 1) / kWavesPerBlock));
#define DDPB_ACC(BF, FI)                                                                                         \
  hipExtLaunchKernelGGL((accumulate_kernel<BF, FI>), agrid, dim3(kBlock), lds_one_per_cu_, s, t0, nullptr, 0,  \
                        d_segs_ + v0, vn, d_grads_, steps, P_, R_, vec_ok_)
      if (sync_step_bf16_) {
        if (sync_step_first_) DDPB_ACC(true, true); else DDPB_ACC(true, false);
      } else {
        if (sync_step_first_) DDPB_ACC(false, true); else DDPB_ACC(false, false);
      }
#undef DDPB_ACC
      HIP_OK(hipGetLastError(), "launch accumulate_kernel");
      t0 = nullptr;                            // the bucket's start is the accumulation's
    }
    const Segment* segs = (view ? d_view_segs_ : d_segs_) + s0;
    float* const* table = view ? d_view_bases_ : d_grads_;
    const int32_t tp = view ? 1 : P_;
    const uint8_t* used = used_active_ ? d_used_ : nullptr;
    int64_t* stamp = (flags_ & 1) ? d_stamps_ + static_cast<int64_t>(b) * 4 : nullptr;
    int64_t blocks = (nseg + kWavesPerBlock - 1) / kWavesPerBlock;
    if (max_blocks_ > 0) blocks = std::min<int64_t>(blocks, max_blocks_);
    const dim3 grid(static_cast<unsigned>(blocks));
    const dim3 block(kBlock);
    if (mode_ == kModeFused || mode_ == kModeBucketView) {
      const bool compact = (used == nullptr) && wg_per_cu_ != 1;
      switch (R_) {
#define DDPB_FUSED_CASE(RR)                                                                                      \
  case RR:                                                                                                       \
    if (!compact)                                                                                                \
      hipExtLaunchKernelGGL((fused_mean_kernel<RR, true>), grid, block, lds_reserve_, s, t0, t1, 0, segs, nseg,  \
                            table, tp, scale_, vec_ok_, used, zero_unused, stamp);                               \
    else                                                                                                         \
      hipExtLaunchKernelGGL((fused_mean_kernel<RR, false>), grid, block, lds_reserve_, s, t0, t1, 0, segs,      \
                            nseg, table, tp, scale_, vec_ok_, used, zero_unused, stamp);                         \
    break;
        DDPB_FUSED_CASE(1) DDPB_FUSED_CASE(2) DDPB_FUSED_CASE(3) DDPB_FUSED_CASE(4)
        DDPB_FUSED_CASE(5) DDPB_FUSED_CASE(6) DDPB_FUSED_CASE(7) DDPB_FUSED_CASE(8)
        DDPB_FUSED_CASE(9) DDPB_FUSED_CASE(10) DDPB_FUSED_CASE(11) DDPB_FUSED_CASE(12)
        DDPB_FUSED_CASE(13) DDPB_FUSED_CASE(14) DDPB_FUSED_CASE(15) DDPB_FUSED_CASE(16)
#undef DDPB_FUSED_CASE
        default:
          hipExtLaunchKernelGGL(fused_mean_kernel_rt, grid, block, lds_reserve_, s, t0, t1, 0, segs, nseg, table, tp,
                                R_, scale_, pow2_ ? 1 : 0, vec_ok_, used, zero_unused, stamp);
      }
      HIP_OK(hipGetLastError(), "launch fused_mean_kernel");
      return kOk;
    }
    // staged: pack, mean, copy-back on the same side stream
    const int64_t fbase = plan_->flat_base[b];
    const int64_t n = plan_->bucket_elems[b];
    const int64_t stride = plan_->flat_elems;
    hipExtLaunchKernelGGL(pack_kernel, grid, block, lds_reserve_, s, t0, nullptr, 0, segs, nseg, d_grads_, P_, R_, flat_,
                          stride, fbase, vec_ok_, used, stamp);
    HIP_OK(hipGetLastError(), "launch pack_kernel");
    const int64_t n4 = std::max<int64_t>(n >> 2, 1);
    int64_t mblocks = std::min<int64_t>((n4 + kBlock - 1) / kBlock, 2048);
    if (max_blocks_ > 0) mblocks = std::min<int64_t>(mblocks, max_blocks_);
    const dim3 mgrid(static_cast<unsigned>(mblocks));
    switch (R_) {
#define DDPB_MEAN_CASE(RR)                                                                                     \
  case RR:                                                                                                     \
    hipLaunchKernelGGL((mean_kernel<RR>), mgrid, block, lds_reserve_, s, flat_, stride, fbase, n, avg_, scale_, \
                       nullptr);                                                                               \
    break;
      DDPB_MEAN_CASE(1) DDPB_MEAN_CASE(2) DDPB_MEAN_CASE(3) DDPB_MEAN_CASE(4)
      DDPB_MEAN_CASE(5) DDPB_MEAN_CASE(6) DDPB_MEAN_CASE(7) DDPB_MEAN_CASE(8)
      DDPB_MEAN_CASE(9) DDPB_MEAN_CASE(10) DDPB_MEAN_CASE(11) DDPB_MEAN_CASE(12)
      DDPB_MEAN_CASE(13) DDPB_MEAN_CASE(14) DDPB_MEAN_CASE(15) DDPB_MEAN_CASE(16)
#undef DDPB_MEAN_CASE
      default:
        hipLaunchKernelGGL(mean_kernel_rt, mgrid, block, lds_reserve_, s, flat_, stride, fbase, n, avg_, R_, scale_,
                           pow2_ ? 1 : 0, nullptr);
    }
    HIP_OK(hipGetLastError(), "launch mean_kernel");
    hipExtLaunchKernelGGL(copyback_kernel, grid, block, lds_reserve_, s, nullptr, t1, 0, segs, nseg, d_grads_, P_, R_,
                          avg_, fbase, vec_ok_, used, static_cast<int64_t*>(nullptr));
    HIP_OK(hipGetLastError(), "launch copyback_kernel");
    return kOk;
  }

  // A CU holds at most n of the library's workgroups when each reserves more
  // than 1/(n + 1) of the CU's LDS (the kernels use none). The reduction
  // kernels on the side streams follow wg_per_cu_; the accumulation kernel
  // always runs one workgroup per CU (bf16 add on BERT-base shapes, R = 16:
  // 6.0 TB/s against 5.2 at its register-bound eight waves per SIMD).
  int update_lds_reserve(std::string* err) {
    lds_reserve_ = 0;
    lds_one_per_cu_ = 0;
    if (plan_ == nullptr) return kOk;                         // (computed again at bind)
    int per_cu = 0, per_block = 0;
    HIP_OK(hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, device_),
           "LDS per CU");
    HIP_OK(hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, device_),
           "LDS per workgroup");
    // a CU holds at least what one workgroup may use (gfx950: 160 KiB both)
    const size_t cu_lds = static_cast<size_t>(std::max(per_cu, per_block));
    auto reserve = [&](int n) {
      const size_t want = (cu_lds / (n + 1) + 256 + 255) / 256 * 256;
      return std::min<size_t>(want, static_cast<size_t>(per_block));
    };
    lds_one_per_cu_ = reserve(1);
    if (wg_per_cu_ > 0) lds_reserve_ = reserve(wg_per_cu_);
    return kOk;
  }

  void release() {
    if (static_) {                 // the tables live in `scratch`: nothing to free
      {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (g_scratch_owner[device_] == this) g_scratch_owner[device_] = nullptr;
      }
      static_ = false;
      d_grads_ = nullptr;
      d_segs_ = nullptr;
      flat_ = nullptr;
      avg_ = nullptr;
    }
    for (auto e : ev_ready_) if (e) (void)hipEventDestroy(e);
    for (auto e : ev_done_) if (e) (void)hipEventDestroy(e);
    for (auto e : ev_tail_) if (e) (void)hipEventDestroy(e);
    ev_tail_.clear();
    tail_evt_.clear();
    for (auto e : ev_slot_) if (e) (void)hipEventDestroy(e);
    for (auto e : ev_t0_) if (e) (void)hipEventDestroy(e);
    for (auto e : ev_t1_) if (e) (void)hipEventDestroy(e);
    ev_ready_.clear();
    ev_done_.clear();
    ev_slot_.clear();
    ev_t0_.clear();
    ev_t1_.clear();
    if (d_grads_) (void)hipFree(d_grads_);
    if (d_segs_) (void)hipFree(d_segs_);
    if (d_stamps_) (void)hipFree(d_stamps_);
    if (d_steps_) (void)hipFree(d_steps_);
    if (d_view_bases_) (void)hipFree(d_view_bases_);
    if (d_view_segs_) (void)hipFree(d_view_segs_);
    d_view_bases_ = nullptr;
    d_view_segs_ = nullptr;
    if (h_steps_) (void)hipHostFree(h_steps_);
    if (ev_used_) (void)hipEventDestroy(ev_used_);
    if (ev_sync_steps_) (void)hipEventDestroy(ev_sync_steps_);
    if (d_sync_steps_) (void)hipFree(d_sync_steps_);
    if (h_sync_steps_) (void)hipHostFree(h_sync_steps_);
    ev_sync_steps_ = nullptr;
    d_sync_steps_ = nullptr;
    h_sync_steps_ = nullptr;
    sync_step_active_ = false;
    sync_steps_recorded_ = false;
    if (d_used_) (void)hipFree(d_used_);
    if (h_used_) (void)hipHostFree(h_used_);
    ev_used_ = nullptr;
    d_used_ = nullptr;
    h_used_ = nullptr;
    used_active_ = false;
    used_recorded_ = false;
    d_grads_ = nullptr;
    d_segs_ = nullptr;
    d_stamps_ = nullptr;
    d_steps_ = nullptr;
    h_steps_ = nullptr;
  }

  const Plan* plan_ = nullptr;
  bool static_ = false;        // bound by bind_static: tables in `scratch`
  int32_t R_ = 0, P_ = 0, mode_ = 0, flags_ = 0;
  int device_ = 0;
  bool pow2_ = true;
  float scale_ = 1.0f;
  int32_t vec_ok_ = 1;
  int32_t max_blocks_ = 0;     // cap on workgroups per reduction launch (0 = none)
  int32_t wg_per_cu_ = 1;      // fused-kernel workgroups per CU (0 = no limit)
  size_t lds_reserve_ = 0;     // dynamic LDS per reduction workgroup that enforces it
  size_t lds_one_per_cu_ = 0;  // ... for one workgroup per CU (accumulation)
  hipStream_t compute_ = nullptr;
  std::vector<hipStream_t> side_;
  std::vector<uint8_t> side_used_;
  float** d_grads_ = nullptr;
  Segment* d_segs_ = nullptr;
  int64_t* d_stamps_ = nullptr;
  void** d_steps_ = nullptr;
  float** d_view_bases_ = nullptr;
  Segment* d_view_segs_ = nullptr;
  void** h_steps_ = nullptr;
  uint8_t* d_used_ = nullptr;   // R x P used flags of the coming synchronisation
  uint8_t* h_used_ = nullptr;   // pinned staging for their upload
  hipEvent_t ev_used_ = nullptr;
  bool used_recorded_ = false;
  bool used_active_ = false;
  void** d_sync_steps_ = nullptr;   // R x P step pointers of the synchronising micro-step
  void** h_sync_steps_ = nullptr;   // pinned staging for their upload
  hipEvent_t ev_sync_steps_ = nullptr;
  bool sync_steps_recorded_ = false;
  bool sync_step_active_ = false;
  bool sync_step_bf16_ = false;
  bool sync_step_first_ = false;
  float* flat_ = nullptr;
  float* avg_ = nullptr;
  std::vector<hipEvent_t> ev_ready_, ev_done_, ev_slot_, ev_t0_, ev_t1_, ev_tail_;
  std::vector<hipEvent_t> tail_evt_;         // per side stream: event of its last bucket this iteration
  std::vector<uint8_t> slot_valid_, slot_recorded_;
  int next_slot_ = 0;
};

}  // namespace

std::unique_ptr<Launcher> make_launcher() { return std::make_unique<HipLauncher>(); }

}  // namespace ddpb
