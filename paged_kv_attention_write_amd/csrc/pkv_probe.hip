// Read-bandwidth probe (gfx950): the rate at which this device streams bytes
// from HBM when nothing is computed on them.  It gives the benchmark a
// measured read ceiling to set beside the published 8 TB/s, for two access
// patterns:
//   - one contiguous buffer, split into equal shares, one per workgroup;
//   - the pages of a block pool named by a list of page ids (the pages of a
//     shuffled block table read whole, in list order), split the same way.
// Loads are 16 bytes per lane, non-temporal, four in flight per lane, one
// persistent workgroup of 8 waves per compute unit: the shape the decode
// kernel reads with.  Each workgroup folds what it read into one word and
// stores it, so that no load can be dropped.
//
// This library is measurement plumbing of the benchmark; the attention
// library does not use it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kInFlight = 4;                           // 16-byte loads per lane per step
constexpr int64_t kStepBytes = int64_t(kThreads) * 16 * kInFlight;  // 32 KiB per workgroup step

__device__ __forceinline__ uint32_t fold(u32x4_t v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Bytes [begin, end) of `base` (16-byte aligned, end - begin a multiple of 16).
__device__ __forceinline__ uint32_t read_range(const char* base, int64_t begin, int64_t end) {
    uint32_t acc = 0;
    const int64_t t = threadIdx.x;
    int64_t off = begin;
    for (; off + kStepBytes <= end; off += kStepBytes) {
        u32x4_t v[kInFlight];
#pragma unroll
        for (int i = 0; i < kInFlight; ++i)
            v[i] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4_t*>(base + off + (int64_t(i) * kThreads + t) * 16));
#pragma unroll
        for (int i = 0; i < kInFlight; ++i) acc ^= fold(v[i]);
    }
    for (int64_t o = off + t * 16; o < end; o += int64_t(kThreads) * 16)
        acc ^= fold(__builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(base + o)));
    return acc;
}

__global__ __launch_bounds__(kThreads) void probe_contiguous(const char* __restrict__ base, int64_t units,
                                                             uint32_t* __restrict__ sink) {
    // units of 16 bytes, an equal share per workgroup
    const int64_t per = (units + gridDim.x - 1) / gridDim.x;
    const int64_t u0 = min<int64_t>(units, per * blockIdx.x);
    const int64_t u1 = min<int64_t>(units, u0 + per);
    const uint32_t acc = read_range(base, u0 * 16, u1 * 16);
    __shared__ uint32_t red[kThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t a = 0;
        for (int i = 0; i < kThreads; ++i) a ^= red[i];
        sink[blockIdx.x] = a;
    }
}

__global__ __launch_bounds__(kThreads) void probe_pages(const char* __restrict__ base, int64_t page_bytes,
                                                        int64_t num_pool_pages, const int32_t* __restrict__ pages,
                                                        int64_t num_pages, uint32_t* __restrict__ sink) {
    const int64_t per = (num_pages + gridDim.x - 1) / gridDim.x;
    const int64_t p0 = min<int64_t>(num_pages, per * blockIdx.x);
    const int64_t p1 = min<int64_t>(num_pages, p0 + per);
    uint32_t acc = 0;
    for (int64_t p = p0; p < p1; ++p) {
        // an id outside the pool is clamped into it: every read stays in bounds
        const int64_t id = min<int64_t>(max<int64_t>(pages[p], 0), num_pool_pages - 1);
        acc ^= read_range(base + id * page_bytes, 0, page_bytes);
    }
    __shared__ uint32_t red[kThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t a = 0;
        for (int i = 0; i < kThreads; ++i) a ^= red[i];
        sink[blockIdx.x] = a;
    }
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16) of `base` (16-byte aligned); with `pages`
// non-NULL, read instead the num_pages pages of page_bytes (a multiple of
// 16) each that pages[] names in a pool of num_pool_pages pages at `base`.
// `sink` receives one word per workgroup (blocks words).  Returns 0, or -1
// for bad arguments, -7 for a launch error.
int pkv_probe_read(const void* base, int64_t bytes, const int32_t* pages, int64_t num_pages, int64_t page_bytes,
                   int64_t num_pool_pages, uint32_t* sink, int32_t blocks, void* stream) {
    if (base == nullptr || sink == nullptr || blocks < 1 || (reinterpret_cast<uintptr_t>(base) & 15) != 0) return -1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (pages == nullptr) {
        if (bytes <= 0 || bytes % 16 != 0) return -1;
        hipLaunchKernelGGL(probe_contiguous, dim3(blocks), dim3(kThreads), 0, st, static_cast<const char*>(base),
                           bytes / 16, sink);
    } else {
        if (num_pages <= 0 || page_bytes <= 0 || page_bytes % 16 != 0 || num_pool_pages <= 0) return -1;
        hipLaunchKernelGGL(probe_pages, dim3(blocks), dim3(kThreads), 0, st, static_cast<const char*>(base),
                           page_bytes, num_pool_pages, pages, num_pages, sink);
    }
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"
