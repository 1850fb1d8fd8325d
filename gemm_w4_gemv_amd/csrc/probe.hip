// Measurement-only kernel: a plain streaming read of a device buffer.
//
// It gives the HBM read rate this GPU actually sustains, the ceiling against
// which the weight-streaming kernels are read (the INT4 GEMV reads each
// weight byte once, so its rate can approach this one but not exceed it).
// Each workgroup streams one contiguous region of the buffer: per step its
// four waves read 16 KB in a row (each wave four 1 KB pieces, 16 bytes per
// lane, non-temporal loads, all four in flight), folded with XOR into one
// word per workgroup so no load is dead.  Contiguous per-workgroup streams
// measured 7.0-7.2 TB/s on MI355X (2 GiB, 512-4096 workgroups), against
// 5.8-6.4 TB/s for the same loads spread grid-wide (consecutive steps of a
// workgroup a whole grid apart).  With zero bytes one workgroup writes one
// word: the cost of a launch with no work.
#include "w4_device.hpp"
#include "w4_internal.hpp"

namespace w4 {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocks = 512;        // workgroups for a large buffer
constexpr size_t kProbeMinWords = 4096;  // at least 64 KB per workgroup

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4_t* __restrict__ src, size_t words,
                                                                    size_t per, uint32_t* __restrict__ sink) {
    const size_t begin = per * blockIdx.x;
    const size_t end = begin + per < words ? begin + per : words;
    size_t i = begin + threadIdx.x;
    uint32_t acc = 0u;
    for (; i + 3 * kProbeThreads < end; i += 4 * kProbeThreads) {
        const u32x4_t a = __builtin_nontemporal_load(src + i);
        const u32x4_t b = __builtin_nontemporal_load(src + i + kProbeThreads);
        const u32x4_t c = __builtin_nontemporal_load(src + i + 2 * kProbeThreads);
        const u32x4_t d = __builtin_nontemporal_load(src + i + 3 * kProbeThreads);
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < end; i += kProbeThreads) {
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
    // Up to kProbeBlocks workgroups (at most one digest word each in the sink),
    // each with at least kProbeMinWords words unless the buffer is smaller.
    size_t blocks = (words + kProbeMinWords - 1) / kProbeMinWords;
    if (blocks > (size_t)kProbeBlocks) blocks = kProbeBlocks;
    if (blocks > (size_t)sink_words) blocks = (size_t)sink_words;
    if (blocks == 0) blocks = 1;
    // Words per workgroup, a multiple of one step's 256 lanes.
    size_t per = (words + blocks - 1) / blocks;
    per = (per + kProbeThreads - 1) / kProbeThreads * kProbeThreads;
    read_probe_kernel<<<(unsigned)blocks, kProbeThreads, 0, stream>>>(static_cast<const u32x4_t*>(src), words, per,
                                                                      sink);
    return hipGetLastError();
}

}  // namespace w4
