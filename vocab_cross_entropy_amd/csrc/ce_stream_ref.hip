// Reference streaming pass for the bandwidth figures (ce_stream_reference): not a step of the
// cross-entropy method, a plain one-pass kernel that moves the bytes a fused call moves, so that
// benchmarks can report its rate beside the fused kernel's.
//
// A buffer is streamed in 64 KiB workgroup spans (1024 threads, 4 vectors of 16 bytes a thread, all
// loads in flight before the stores) with the raw buffer loads and stores, non-temporal bit set, that
// the fused kernel streams its logits with.  dst == src: every 32-bit word is XORed with `flip` and
// written back in place (one read and one write of each byte, as in the fused step); otherwise a copy.
// Of the one-pass shapes measured in place over 2.1 GB (256 threads x 4, 8 or 16 vectors, 512 x 8,
// 1024 x 4, and grid-stride loops that load the next span before storing the current one) this one and
// 512 x 8 were the fastest, about 5.9 TB/s.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ce_internal.h"

namespace vce {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRefT = 1024, kRefP = 4;
constexpr int64_t kRefSpan = (int64_t)kRefT * kRefP * 16;
constexpr int kRawWord3 = 0x00020000;  // raw buffer, 32-bit element format
constexpr int kNonTemporal = 2;        // the buffer instructions' cache-policy operand: nt

__global__ __launch_bounds__(kRefT) void k_stream_ref(const char* src, char* dst, int64_t bytes, uint32_t flip) {
  const int64_t base = (int64_t)blockIdx.x * kRefSpan;
  const int64_t left = bytes - base;
  const int span = (int)(left < kRefSpan ? left : kRefSpan);  // a load or store past it is dropped
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src + base), 0, span, kRawWord3);
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(dst + base, 0, span, kRawWord3);
  u32x4 v[kRefP];
#pragma unroll
  for (int j = 0; j < kRefP; ++j)
    v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (j * kRefT + (int)threadIdx.x) * 16, 0, kNonTemporal);
#pragma unroll
  for (int j = 0; j < kRefP; ++j)
    __builtin_amdgcn_raw_buffer_store_b128(v[j] ^ flip, rd, (j * kRefT + (int)threadIdx.x) * 16, 0, kNonTemporal);
}

}  // namespace

hipError_t launch_stream_ref(const void* src, void* dst, int64_t bytes, uint32_t flip, hipStream_t stream,
                             hipEvent_t ev0, hipEvent_t ev1) {
  if (bytes == 0) return hipSuccess;
  hipError_t e = hipSuccess;
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
  const dim3 grid((uint32_t)((bytes + kRefSpan - 1) / kRefSpan));
  hipLaunchKernelGGL(k_stream_ref, grid, dim3(kRefT), 0, stream, static_cast<const char*>(src),
                     static_cast<char*>(dst), bytes, flip);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev1) e = hipEventRecord(ev1, stream);
  return e;
}

}  // namespace vce
