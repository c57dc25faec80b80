// layout.hip -- conversion between plain [N][C][spatial] activations and the
// channel-packed layout [N][ceil(C/g)][spatial][g] (g = one 16-byte vector of
// channels: 8 of a 16-bit type, 4 of fp32; zero past C).
//
// The packed layout is the one the implicit-GEMM kernels stage from: a
// channel group of a pixel is one 16-byte vector, so a halo row of one group
// is a contiguous run of memory that can be copied straight into on-chip
// memory.  The page "SeedVR2 NCNN Vulkan" (section 9) plans to keep its
// channel packing (pack4) through the whole network so that layers stop
// packing and unpacking between each other; the conversions here are for the
// network's edges only.  Both are bound by HBM: one pass over each tensor.
#include "device_common.h"
#include "internal.h"

namespace libconv {
namespace {

constexpr int kThreads = 256;

struct LayoutArgs {
  const void* src;
  void* dst;
  int N, C, S;       // batch, channels, spatial elements per channel (T*H*W)
  int groups;        // ceil(C / SE)
  uint32_t plain_bytes, packed_bytes;
};

// One thread per 16-byte packed vector u = (n, group, s): lanes walk s, so
// each of the SE channel planes is read as a contiguous run across the wave
// and the vectors are written contiguously.
template <int EB>
__global__ __launch_bounds__(kThreads) void pack_act_kernel(LayoutArgs a) {
  constexpr int SE = 16 / EB;
  const long long u = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long total = (long long)a.N * a.groups * a.S;
  if (u >= total) return;
  const int s = (int)(u % a.S);
  const long long ng = u / a.S;
  const int g = (int)(ng % a.groups), n = (int)(ng / a.groups);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.src, a.plain_bytes);
  const __amdgpu_buffer_rsrc_t dr = make_rsrc(a.dst, a.packed_bytes);
  uint32_t e[SE];
#pragma unroll
  for (int j = 0; j < SE; ++j) {
    const int c = g * SE + j;
    const int off = (int)(((long long)n * a.C + c) * a.S + s) * EB;
    e[j] = EB == 4 ? __builtin_amdgcn_raw_buffer_load_b32(sr, guard_offset(c < a.C, off), 0, 0)
                   : __builtin_amdgcn_raw_buffer_load_b16(sr, guard_offset(c < a.C, off), 0, 0);
  }
  u32x4_t v;
#pragma unroll
  for (int m = 0; m < 4; ++m)
    v[m] = EB == 4 ? e[m] : ((e[2 * m] & 0xffffu) | (e[2 * m + 1] << 16));
  __builtin_amdgcn_raw_buffer_store_b128(v, dr, (int)(u * 16), 0, 0);
}

template <int EB>
__global__ __launch_bounds__(kThreads) void unpack_act_kernel(LayoutArgs a) {
  constexpr int SE = 16 / EB;
  const long long u = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long total = (long long)a.N * a.groups * a.S;
  if (u >= total) return;
  const int s = (int)(u % a.S);
  const long long ng = u / a.S;
  const int g = (int)(ng % a.groups), n = (int)(ng / a.groups);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.src, a.packed_bytes);
  const __amdgpu_buffer_rsrc_t dr = make_rsrc(a.dst, a.plain_bytes);
  const u32x4_t v =
      __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sr, (int)(u * 16), 0, 0));
#pragma unroll
  for (int j = 0; j < SE; ++j) {
    const int c = g * SE + j;
    if (c >= a.C) break;
    const int off = (int)(((long long)n * a.C + c) * a.S + s) * EB;
    if constexpr (EB == 4)
      __builtin_amdgcn_raw_buffer_store_b32(v[j], dr, off, 0, 0);
    else
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(v[j / 2] >> (16 * (j & 1))), dr, off, 0, 0);
  }
}

}  // namespace

long long cpack_bytes(int N, int C, long long spatial, int dtype) {
  const int se = 16 / dtype_bytes(dtype);
  return (long long)N * ((C + se - 1) / se) * spatial * 16;
}

libconv_status layout_launch(const void* src, void* dst, int N, int C, long long spatial,
                             int dtype, bool to_packed, hipStream_t stream) {
  LayoutArgs a;
  a.src = src;
  a.dst = dst;
  a.N = N;
  a.C = C;
  a.S = (int)spatial;
  const int eb = dtype_bytes(dtype);
  a.groups = (C + 16 / eb - 1) / (16 / eb);
  a.plain_bytes = (uint32_t)((long long)N * C * spatial * eb);
  a.packed_bytes = (uint32_t)cpack_bytes(N, C, spatial, dtype);
  const long long words = (long long)N * a.groups * spatial;
  if (words == 0) return LIBCONV_OK;
  const unsigned grid = (unsigned)((words + kThreads - 1) / kThreads);
  if (eb == 4) {
    if (to_packed)
      hipLaunchKernelGGL(pack_act_kernel<4>, dim3(grid), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(unpack_act_kernel<4>, dim3(grid), dim3(kThreads), 0, stream, a);
  } else {
    if (to_packed)
      hipLaunchKernelGGL(pack_act_kernel<2>, dim3(grid), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(unpack_act_kernel<2>, dim3(grid), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? LIBCONV_OK : LIBCONV_ERR_LAUNCH;
}

}  // namespace libconv
