// Streaming-read probe: the HBM read bandwidth this chip achieves for the
// two access patterns of the decode step, as the yardstick for the kernels'
// roofline fractions (the vendor peak of 8 TB/s is not reachable by reads).
//
//   linear:  a buffer read front to back in 4 KiB chunks;
//   gather:  the same chunks read in a caller-given order (a random
//            permutation stands for page statistics and K tiles reached
//            through a page table, which arrive in 4 KiB-sized pieces at
//            random physical pages).
//
// A 256-thread block reads one chunk per step with one 16-byte load per
// thread, UNROLL chunks in flight, blocks striding over the chunk list.  The
// loaded words are folded into one value per thread, which is stored only
// when it equals a constant the data would have to hit by chance, so the
// loads stay live without a store stream of their own.
#include "ekv_device.h"
#include "ekv_internal.h"

namespace ekv {

constexpr int kProbeThreads = 256;
constexpr int kProbeChunk = kProbeThreads * 16;   // bytes per chunk (4 KiB)

template <int UNROLL>
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const uint4* __restrict__ buf, long n_chunks,
                                                                  const int32_t* __restrict__ order,
                                                                  uint32_t* __restrict__ sink) {
    constexpr int W = kProbeChunk / 16;           // uint4 per chunk
    uint32_t acc = 0;
    const long stride = (long)gridDim.x * UNROLL;
    for (long c0 = (long)blockIdx.x * UNROLL; c0 < n_chunks; c0 += stride) {
        uint4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const long c = c0 + u < n_chunks ? c0 + u : c0;       // past the end: re-read c0 (ignored)
            long ch = order ? (long)order[c] : c;
            ch = (ch >= 0 && ch < n_chunks) ? ch : 0;               // a bad order entry reads chunk 0
            v[u] = buf[ch * W + threadIdx.x];
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            if (c0 + u < n_chunks) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

hipError_t launch_probe_read(const void* buf, long n_chunks, const int32_t* order, int unroll, int blocks,
                             uint32_t* sink, hipStream_t s) {
    const dim3 grid(blocks), block(kProbeThreads);
    switch (unroll) {
        case 2: probe_read_kernel<2><<<grid, block, 0, s>>>((const uint4*)buf, n_chunks, order, sink); break;
        case 4: probe_read_kernel<4><<<grid, block, 0, s>>>((const uint4*)buf, n_chunks, order, sink); break;
        case 8: probe_read_kernel<8><<<grid, block, 0, s>>>((const uint4*)buf, n_chunks, order, sink); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ekv
