// Read-bandwidth probe: stream a device buffer with 16-byte loads and keep
// nothing but a running XOR, so the achievable HBM read rate of the device can
// be measured beside the decode scan, which is itself a read-only stream of
// the packed cache.  Decode is bound by memory bandwidth (the llama.cpp fork's
// README, "TurboQuant KV 캐시 압축 for llama.cpp", v1.8.0 "성능 특성": decode
// reads the weights from memory every token), so this rate is the practical
// ceiling the scan is compared with.
#include <hip/hip_runtime.h>

#include "tq.h"

namespace {

constexpr int kUnroll = 8;    // 16-byte loads in flight per thread
constexpr int kThreads = 512;  // one block of 8 waves per compute unit

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte load: the data is read once, so it should
// not displace anything in the caches.
__device__ __forceinline__ uint32_t load_xor(const uint4* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return v[0] ^ v[1] ^ v[2] ^ v[3];
}

// Measured on MI355X over 1 GiB: one block of 8 waves per compute unit with
// 8 non-temporal loads in flight per lane reads fastest (about 6.9 TB/s); 4 or
// 8 blocks per unit, or plain loads, read 5.1-6.4 TB/s.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                               uint32_t* sink) {
    const int64_t nt = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kUnroll - 1) * nt < n16; i += kUnroll * nt) {
        uint32_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = load_xor(src + i + u * nt);  // all issued before any use
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; i < n16; i += nt) acc ^= load_xor(src + i);
    // the loads feed a branch, so they stay; the store almost never happens
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

extern "C" int tq_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    if (!src || !sink || ((uintptr_t)src % 16) != 0 || ((uintptr_t)sink % 4) != 0 || bytes % 16 != 0)
        return TQ_EINVAL;
    if (bytes == 0) return TQ_OK;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const int64_t n16 = (int64_t)(bytes / 16);
    int64_t blocks = cus;
    const int64_t need = (n16 + kThreads - 1) / kThreads;
    if (blocks > need) blocks = need;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream,
                       static_cast<const uint4*>(src), n16, sink);
    return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EDEVICE;
}
