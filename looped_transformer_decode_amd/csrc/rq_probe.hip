// rq_stream_read: a plain streaming read of a device buffer, as a measuring stick.
//
// Two workgroups per CU each read one contiguous slab with 16-byte non-temporal loads (the
// hint that reads a once-read stream fastest here), eight in flight per thread, and fold
// them with XOR into one word per thread (written to `sink` so the loads cannot be
// dropped).  Two long slabs per CU read 4% faster than about sixteen shorter ones (6.66
// against 6.39 TB/s over 478 MB of cold replicas).  It holds none of the method's arithmetic.  Timed over the
// same buffers as the decode kernel, it shows the read rate that a simple load loop
// reaches on the device, next to the datasheet peak.
#include "rq_common.hpp"

namespace rq {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr int kProbeMaxBlocks = 4096;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* __restrict__ p, int64_t n,
                                                                    int64_t per, uint32_t* __restrict__ sink) {
    const int64_t beg = (int64_t)blockIdx.x * per;
    const int64_t end = beg + per < n ? beg + per : n;
    uint32_t acc = 0;
    for (int64_t i = beg + threadIdx.x; i < end; i += kProbeThreads * kProbeUnroll) {
        uint4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const int64_t k = i + (int64_t)u * kProbeThreads;
            if (k < end) {
                typedef uint32_t nt4 __attribute__((ext_vector_type(4)));
                const nt4 t = __builtin_nontemporal_load(reinterpret_cast<const nt4*>(p + k));
                v[u] = uint4{t.x, t.y, t.z, t.w};
            } else {
                v[u] = uint4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    sink[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace rq

using namespace rq;

extern "C" rq_status rq_stream_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                                    hipStream_t stream) {
    if (!buf || !sink || bytes == 0 || bytes % 16 != 0) return RQ_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(buf) & 15u) return RQ_ERR_MISALIGNED;
    if (sink_words < (size_t)kProbeMaxBlocks * kProbeThreads) return RQ_ERR_WORKSPACE;
    const int64_t n = (int64_t)(bytes / 16);
    // two workgroups per CU
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || cus <= 0)
        cus = 256;
    int64_t nb = 2 * (int64_t)cus;
    nb = nb > kProbeMaxBlocks ? kProbeMaxBlocks : nb;
    const int64_t chunk = (int64_t)kProbeThreads * kProbeUnroll;
    int64_t per = (n + nb - 1) / nb;
    per = (per + chunk - 1) / chunk * chunk;
    nb = (n + per - 1) / per;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)nb), dim3(kProbeThreads), 0, stream,
                       static_cast<const uint4*>(buf), n, per, sink);
    return hipGetLastError() == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}
