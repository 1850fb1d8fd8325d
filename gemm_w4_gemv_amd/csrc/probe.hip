// Measurement-only kernel: a plain streaming read of a device buffer.
//
// It gives the HBM read rate this GPU actually sustains, the ceiling against
// which the weight-streaming kernels are read (the INT4 GEMV reads each
// weight byte once, so its rate can approach this one but not exceed it).
// Each thread reads 16-byte words at a grid-wide stride with non-temporal
// loads, four in flight, and folds them with XOR into one word per
// workgroup, so no load is dead.  With zero bytes one workgroup writes one
// word: the cost of a launch with no work.
#include "w4_device.hpp"
#include "w4_internal.hpp"

namespace w4 {
namespace {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4_t* __restrict__ src, size_t words,
                                                                    uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * kProbeThreads;
    size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
    uint32_t acc = 0u;
    for (; i + 3 * stride < words; i += 4 * stride) {
        const u32x4_t a = __builtin_nontemporal_load(src + i);
        const u32x4_t b = __builtin_nontemporal_load(src + i + stride);
        const u32x4_t c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4_t d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < words; i += stride) {
        const u32x4_t a = __builtin_nontemporal_load(src + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    // Fold the workgroup's words into one (no load may be optimised away).
    __shared__ uint32_t red[kProbeThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int h = kProbeThreads / 2; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] ^= red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

}  // namespace

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int sink_words, hipStream_t stream) {
    const size_t words = bytes / 16;
    // Enough workgroups to fill every compute unit several times, bounded by the sink.
    const size_t want = (words + kProbeThreads - 1) / kProbeThreads;
    const unsigned blocks = (unsigned)(want == 0 ? 1 : (want < (size_t)sink_words ? want : (size_t)sink_words));
    read_probe_kernel<<<blocks, kProbeThreads, 0, stream>>>(static_cast<const u32x4_t*>(src), words, sink);
    return hipGetLastError();
}

}  // namespace w4
