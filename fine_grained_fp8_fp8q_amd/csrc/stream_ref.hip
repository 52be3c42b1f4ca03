// A plain streaming kernel with the quantizers' traffic mix: 2 bytes read and
// 1 byte written per element (the high byte of each 16-bit input), 16-byte
// non-temporal accesses, one pass (one thread per 16 elements).  It is a
// measuring stick, not part of the quantization path: the bench times it over
// the same number of elements as a quantizer to give the rate a bare stream
// of those bytes reaches on the same GPU.  Built into its own library
// (libfp8q_streamref.so); libfp8q.so does not contain it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_2to1_kernel(const v4u* __restrict__ x, v4u* __restrict__ y,
                                                          int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const v4u a = __builtin_nontemporal_load(&x[2 * i]);
  const v4u b = __builtin_nontemporal_load(&x[2 * i + 1]);
  v4u o;
  o.x = __builtin_amdgcn_perm(a.y, a.x, 0x07050301u);
  o.y = __builtin_amdgcn_perm(a.w, a.z, 0x07050301u);
  o.z = __builtin_amdgcn_perm(b.y, b.x, 0x07050301u);
  o.w = __builtin_amdgcn_perm(b.w, b.z, 0x07050301u);
  __builtin_nontemporal_store(o, &y[i]);
}

}  // namespace

// x: device, 2 * n_elems bytes; y: device, n_elems bytes; both 16-byte
// aligned; n_elems a multiple of 16 and below 2^40.  Returns 0, 1 for bad
// arguments (nothing launched) or the HIP error of the launch.
extern "C" int fp8q_streamref_2to1(const void* x, void* y, int64_t n_elems, hipStream_t stream) {
  if (n_elems < 0 || n_elems % 16 != 0 || n_elems >= (int64_t(1) << 40) ||
      (reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) % 16 != 0) {
    return 1;
  }
  const int64_t n16 = n_elems / 16;
  if (n16 == 0) return 0;
  hipLaunchKernelGGL(stream_2to1_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const v4u*>(x), static_cast<v4u*>(y), n16);
  return (int)hipGetLastError();
}
