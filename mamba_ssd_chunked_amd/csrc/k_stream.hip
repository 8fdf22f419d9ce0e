// Benchmark instrumentation: the HBM rate a plain streaming kernel reaches on this GPU for a
// given mix of reads and writes.  The chunk kernels' algorithmic bytes are mostly reads with a
// share of writes (the state kernel about 3:1, the backward target kernel about 4:1, the K4
// passes 1:1), and HBM3E delivers less than its nominal 8 TB/s to such mixes; this measures
// what a kernel that does nothing but move those bytes gets, so that each kernel's rate can
// be compared with the rate its own mix allows.
//
// k_stream<NR, NW, NTL>: NR source arrays and NW destination arrays of n float4 each
// (contiguous, array a at offset a * n); every work-item of a grid-stride loop reads its
// float4 from each source, sums them and writes the sum to each destination (with NW = 0 a
// never-taken store keeps the loads alive).  NTL = true makes the loads and stores
// non-temporal.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

template <int NR, int NW, bool NTL>
__global__ __launch_bounds__(NT) void k_stream(const v4f* __restrict__ src, v4f* __restrict__ dst,
                                               int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * NT;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x; i < n; i += stride) {
        v4f s = zero4();
#pragma unroll
        for (int a = 0; a < NR; ++a) {
            const v4f* p = src + a * n + i;
            s += NTL ? __builtin_nontemporal_load(p) : *p;
        }
#pragma unroll
        for (int a = 0; a < NW; ++a) {
            v4f* q = dst + a * n + i;
            if (NTL)
                __builtin_nontemporal_store(s, q);
            else
                *q = s;
        }
        if (NW == 0 && s[0] == 1.0e30f) dst[i] = s;  // never true for the probe's zero inputs
    }
}

hipError_t launch_stream_probe(int reads, int writes, bool nontemporal, const void* src, void* dst,
                               int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    // 16 workgroups per CU of grid-stride work: enough loads in flight to cover the latency
    const int64_t need = (n + NT - 1) / NT;
    const dim3 grid(static_cast<unsigned>(need < 4096 ? need : 4096));
    const v4f* s = static_cast<const v4f*>(src);
    v4f* d = static_cast<v4f*>(dst);
#define X(R_, W_)                                                                            \
    if (reads == R_ && writes == W_) {                                                       \
        if (nontemporal)                                                                     \
            hipLaunchKernelGGL((k_stream<R_, W_, true>), grid, dim3(NT), 0, st, s, d, n);    \
        else                                                                                 \
            hipLaunchKernelGGL((k_stream<R_, W_, false>), grid, dim3(NT), 0, st, s, d, n);   \
        return hipGetLastError();                                                            \
    }
    X(1, 0) X(6, 1) X(4, 1) X(3, 1) X(2, 1) X(1, 1) X(0, 1)
#undef X
    return hipErrorInvalidValue;
}

}  // namespace ssd
