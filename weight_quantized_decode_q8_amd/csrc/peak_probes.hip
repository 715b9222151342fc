// peak_probes.hip -- measurement kernels, not part of the product path:
// the achievable HBM read rate and matrix-core rate of the GPU they run on,
// and its shader clock under matrix-core load.  The rooflines of the
// library's kernels are quoted against the published peaks; these give the
// rates a kernel can actually reach on the same chip, next to them.
//
//  - stream_read_kernel: every lane reads 16-byte pieces, 4, 8 or 16 in flight,
//    with non-temporal loads (the loads the GEMVs use), over a buffer far
//    larger than the caches.  The pieces are folded into one value that is
//    stored only when it equals a sentinel the host picks (never, in
//    practice), so the loads cannot be optimised away and nothing is
//    written.
//  - mfma_loop_kernel: kChains independent accumulators per wave, each
//    updated iters times by v_mfma_i32_16x16x64_i8 (kind 0) or
//    v_mfma_f32_16x16x32_f16 (kind 1) on register operands: the matrix
//    pipe's issue rate with no memory traffic.  Wave 0 of workgroup 0
//    records the shader-clock count (s_memtime) and the constant-rate
//    wall-clock count (s_memrealtime) around its loop, which gives the
//    clock.
//  - mfma_valu_kernel: 8 independent int8 MFMA chains per wave, each MFMA
//    followed (by scheduling-group barriers) by a fixed number of
//    independent f32 FMAs, or either kind alone: whether the vector ALU's
//    work hides behind the matrix pipe's on this chip or adds to it.
//  - lds_read_kernel: every lane reads 4, 8 or 16 bytes of LDS per
//    instruction, consecutive lanes at consecutive addresses (no bank
//    conflicts): the LDS read rate per CU.
#include <hip/hip_runtime.h>

#include "qg_internal.h"
#include "qgemv_probes.h"

namespace qg {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kStreamThreads = 512;

template <int kLoads>
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const i32x4 *__restrict__ p, size_t n,
                                                                     unsigned sentinel, unsigned *sink) {
  const size_t stride = (size_t)gridDim.x * kStreamThreads;
  size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
  unsigned acc = 0;
  for (; i + (kLoads - 1) * stride < n; i += kLoads * stride) {
    i32x4 v[kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; k++) v[k] = __builtin_nontemporal_load(p + i + k * stride);
#pragma unroll
    for (int k = 0; k < kLoads; k++) acc ^= (unsigned)(v[k].x ^ v[k].y ^ v[k].z ^ v[k].w);
  }
  for (; i < n; i += stride) {
    const i32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= (unsigned)(v.x ^ v.y ^ v.z ^ v.w);
  }
  if (acc == sentinel) sink[blockIdx.x] = acc;
}

constexpr int kChains = 8;

template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float *sink, unsigned long long *clocks) {
  const int lane = threadIdx.x & 63;
  unsigned long long t0 = 0, r0 = 0;
  const bool timer = blockIdx.x == 0 && threadIdx.x < 64;
  if (timer) {
    t0 = clock64();
    r0 = wall_clock64();
  }
  float out = 0.0f;
  if (KIND == 0) {
    i32x4 a = {lane, lane * 3, lane ^ 5, 7}, b = {lane + 1, 2, lane * 5, 9};
    i32x4 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; c++) acc[c] = i32x4{lane + c, 3 * lane + c + 1, 5 * lane + 2 * c + 2, 7 * lane + 3 * c + 3};
    for (int it = 0; it < iters; it++) {
#pragma unroll
      for (int c = 0; c < kChains; c++) acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kChains; c++) out += (float)(acc[c].x + acc[c].y + acc[c].z + acc[c].w);
  } else {
    f16x8 a, b;
#pragma unroll
    for (int k = 0; k < 8; k++) {
      a[k] = (_Float16)((lane + k) & 7);
      b[k] = (_Float16)((lane * 3 + k) & 3);
    }
    f32x4 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; c++) acc[c] = f32x4{(float)(lane + c), (float)(3 * lane + c + 1), (float)(5 * lane + 2 * c + 2), (float)(7 * lane + 3 * c + 3)};
    for (int it = 0; it < iters; it++) {
#pragma unroll
      for (int c = 0; c < kChains; c++) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kChains; c++) out += acc[c].x + acc[c].y + acc[c].z + acc[c].w;
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = out;
  if (timer && lane == 0) {
    clocks[0] = clock64() - t0;
    clocks[1] = wall_clock64() - r0;
  }
}

constexpr int kMvChains = 8;
constexpr int kMvFloats = 32;

// MF: issue the MFMAs; NF: f32 FMAs per MFMA slot (0, 2, 4 or 8).
template <bool MF, int NF>
__global__ __launch_bounds__(1024) void mfma_valu_kernel(int iters, float *sink) {
  const int lane = threadIdx.x & 63;
  const i32x4 a = {lane, lane * 3, lane ^ 5, 7}, b = {lane + 1, 2, lane * 5, 9};
  i32x4 acc[kMvChains];
#pragma unroll
  for (int c = 0; c < kMvChains; c++)
    acc[c] = i32x4{lane + c, 3 * lane + c + 1, 5 * lane + 2 * c + 2, 7 * lane + 3 * c + 3};
  float f[kMvFloats];
#pragma unroll
  for (int j = 0; j < kMvFloats; j++) f[j] = (float)(lane + j) * 0.001f;
  const float x = 1.0001f + lane * 1e-7f;
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int c = 0; c < kMvChains; c++) {
      if (MF) acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[c], 0, 0, 0);
#pragma unroll
      for (int k = 0; k < NF; k++) {
        const int j = (c * NF + k) % kMvFloats;
        f[j] = fmaf(f[j], x, 0.5f);
      }
    }
    // one MFMA, then its FMAs, in program order (not clustered by the
    // scheduler)
#pragma unroll
    for (int c = 0; c < kMvChains; c++) {
      __builtin_amdgcn_sched_group_barrier(0x008, MF ? 1 : 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, NF, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kMvChains; c++) s += (float)(acc[c].x + acc[c].y + acc[c].z + acc[c].w);
#pragma unroll
  for (int j = 0; j < kMvFloats; j++) s += f[j];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

constexpr int kLdsProbeBytes = 65536;

template <int W>
__global__ __launch_bounds__(1024) void lds_read_kernel(int iters, int *sink) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsProbeBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kLdsProbeBytes / 4; i += blockDim.x) reinterpret_cast<int *>(lds)[i] = i * 7;
  __syncthreads();
  int acc = 0;
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      // W bytes per lane at consecutive addresses, wrapped inside the buffer
      const int o = ((((wave * 8 + k) * 64 + lane) * W) + it * 64) & (kLdsProbeBytes - W);
      if (W == 16) {
        const i32x4 v = *reinterpret_cast<const i32x4 *>(lds + o);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
      } else if (W == 8) {
        const int2 v = *reinterpret_cast<const int2 *>(lds + o);
        acc ^= v.x ^ v.y;
      } else {
        acc ^= *reinterpret_cast<const int *>(lds + o);
      }
    }
  }
  sink[(size_t)blockIdx.x * blockDim.x + tid] = acc;
}

}  // namespace
}  // namespace qg

using namespace qg;

extern "C" {

qg_status qg_probe_stream_read(const void *buf, size_t bytes, unsigned sentinel, unsigned *sink, int workgroups,
                               int loads, void *stream) {
  if (!buf || !sink || bytes < 16 || workgroups < 1 || workgroups > (1 << 20) ||
      (reinterpret_cast<uintptr_t>(buf) & 15) || (loads != 4 && loads != 8 && loads != 16))
    return fail(QG_EINVAL, "qg_probe_stream_read: bad argument");
  const i32x4 *p = reinterpret_cast<const i32x4 *>(buf);
  const hipStream_t s = (hipStream_t)stream;
  if (loads == 4)
    stream_read_kernel<4><<<workgroups, kStreamThreads, 0, s>>>(p, bytes / 16, sentinel, sink);
  else if (loads == 8)
    stream_read_kernel<8><<<workgroups, kStreamThreads, 0, s>>>(p, bytes / 16, sentinel, sink);
  else
    stream_read_kernel<16><<<workgroups, kStreamThreads, 0, s>>>(p, bytes / 16, sentinel, sink);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? QG_OK : fail(QG_ELAUNCH, "qg_probe_stream_read: %s", hipGetErrorString(e));
}

qg_status qg_probe_mfma(int kind, int iters, int workgroups, float *sink, unsigned long long *clocks, void *stream) {
  if ((kind != 0 && kind != 1) || iters < 1 || workgroups < 1 || workgroups > (1 << 16) || !sink || !clocks ||
      (reinterpret_cast<uintptr_t>(clocks) & 7) || (reinterpret_cast<uintptr_t>(sink) & 3))
    return fail(QG_EINVAL, "qg_probe_mfma: bad argument");
  if (kind == 0)
    mfma_loop_kernel<0><<<workgroups, 256, 0, (hipStream_t)stream>>>(iters, sink, clocks);
  else
    mfma_loop_kernel<1><<<workgroups, 256, 0, (hipStream_t)stream>>>(iters, sink, clocks);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? QG_OK : fail(QG_ELAUNCH, "qg_probe_mfma: %s", hipGetErrorString(e));
}

qg_status qg_probe_mfma_valu(int mfma, int fmas, int iters, int workgroups, int waves_per_simd, float *sink,
                             size_t sink_elems, void *stream) {
  if ((mfma != 0 && mfma != 1) || (fmas != 0 && fmas != 2 && fmas != 4 && fmas != 8) || (!mfma && !fmas) ||
      iters < 1 || workgroups < 1 || workgroups > (1 << 16) || waves_per_simd < 1 || waves_per_simd > 4 || !sink ||
      (reinterpret_cast<uintptr_t>(sink) & 3) || sink_elems < (size_t)workgroups * 256 * waves_per_simd)
    return fail(QG_EINVAL, "qg_probe_mfma_valu: bad argument");
  const dim3 grid(workgroups), block(256 * waves_per_simd);
  const hipStream_t s = (hipStream_t)stream;
#define QG_MV(M, N) \
  if (mfma == M && fmas == N) mfma_valu_kernel<M, N><<<grid, block, 0, s>>>(iters, sink);
  QG_MV(1, 0) QG_MV(1, 2) QG_MV(1, 4) QG_MV(1, 8) QG_MV(0, 2) QG_MV(0, 4) QG_MV(0, 8)
#undef QG_MV
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? QG_OK : fail(QG_ELAUNCH, "qg_probe_mfma_valu: %s", hipGetErrorString(e));
}

qg_status qg_probe_lds_read(int bytes_per_lane, int iters, int workgroups, int waves, int *sink, size_t sink_elems,
                            void *stream) {
  if ((bytes_per_lane != 4 && bytes_per_lane != 8 && bytes_per_lane != 16) || iters < 1 || workgroups < 1 ||
      workgroups > (1 << 16) || waves < 1 || waves > 16 || !sink || (reinterpret_cast<uintptr_t>(sink) & 3) ||
      sink_elems < (size_t)workgroups * 64 * waves)
    return fail(QG_EINVAL, "qg_probe_lds_read: bad argument");
  const dim3 grid(workgroups), block(64 * waves);
  const hipStream_t s = (hipStream_t)stream;
  if (bytes_per_lane == 16)
    lds_read_kernel<16><<<grid, block, 0, s>>>(iters, sink);
  else if (bytes_per_lane == 8)
    lds_read_kernel<8><<<grid, block, 0, s>>>(iters, sink);
  else
    lds_read_kernel<4><<<grid, block, 0, s>>>(iters, sink);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? QG_OK : fail(QG_ELAUNCH, "qg_probe_lds_read: %s", hipGetErrorString(e));
}

qg_status qg_probe_wall_clock_khz(int *khz) {
  if (!khz) return fail(QG_EINVAL, "qg_probe_wall_clock_khz: null pointer");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev);
  return e == hipSuccess ? QG_OK : fail(QG_ELAUNCH, "qg_probe_wall_clock_khz: %s", hipGetErrorString(e));
}

}  // extern "C"
