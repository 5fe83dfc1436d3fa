// Streaming-read calibration for the HBM roofline (a standalone program, not
// part of libspecverify.so).  Two read-only kernels over buffers far larger
// than the 256 MB Infinity Cache report the read bandwidth one MI355X
// actually sustains, the yardstick beside the nominal 8 TB/s:
//   flat: each workgroup streams one contiguous range, four 16-byte loads
//         per lane per step, two steps in flight (register double buffer);
//   kv  : the attention kernels' access shape -- one wavefront per workgroup
//         walks 32-row blocks of two separate 256-byte-row tensors (K and V,
//         one block of each prefetched ahead), eight 128-byte lines of K per
//         load instruction and four whole rows of V.
// Both run twice: with plain loads and with the non-temporal hint (nt), which
// streams faster on this chip.
// Every workgroup's range lies inside the buffers (checked on the host before
// each launch).  Output: one JSON line with the best rate of each kernel.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

typedef unsigned U4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ U4 ld(const U4* p) {
    return NT ? __builtin_nontemporal_load(p) : *p;
}

constexpr int kFlatU = 4;  // 16-byte loads per lane per step

template <bool NT>
__global__ __launch_bounds__(64) void flat_read(const U4* __restrict__ buf, size_t per_wg, unsigned* out) {
    const U4* p = buf + blockIdx.x * per_wg + threadIdx.x;
    const size_t steps = per_wg / (64 * kFlatU);  // even, >= 2
    U4 a[kFlatU], b[kFlatU];
    unsigned acc = 0;
#pragma unroll
    for (int u = 0; u < kFlatU; ++u) a[u] = ld<NT>(p + u * 64);
    for (size_t i = 0; i < steps; i += 2) {
        const size_t nb = (i + 1) * 64 * kFlatU;
#pragma unroll
        for (int u = 0; u < kFlatU; ++u) b[u] = ld<NT>(p + nb + u * 64);
#pragma unroll
        for (int u = 0; u < kFlatU; ++u) acc ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w;
        const size_t na = (i + 2 < steps ? i + 2 : i) * 64 * kFlatU;
#pragma unroll
        for (int u = 0; u < kFlatU; ++u) a[u] = ld<NT>(p + na + u * 64);
#pragma unroll
        for (int u = 0; u < kFlatU; ++u) acc ^= b[u].x ^ b[u].y ^ b[u].z ^ b[u].w;
    }
    out[blockIdx.x * 64 + threadIdx.x] = acc;
}

// One 32-row block of K and V (rows of 16 chunks of 16 bytes).
template <bool NT>
__device__ __forceinline__ void kv_block(U4 (&kf)[8], U4 (&vr)[8], const U4* K, const U4* V, long row0, int lane) {
#pragma unroll
    for (int i = 0; i < 8; ++i) kf[i] = ld<NT>(K + (row0 + 8 * (i >> 1) + (lane >> 3)) * 16 + (i & 1) * 8 + (lane & 7));
#pragma unroll
    for (int j = 0; j < 8; ++j) vr[j] = ld<NT>(V + (row0 + 8 * (lane >> 4) + j) * 16 + (lane & 15));
}

template <bool NT>
__global__ __launch_bounds__(64) void kv_read(const U4* __restrict__ K, const U4* __restrict__ V, long blocks_per_wg,
                                              unsigned* out) {
    const int lane = threadIdx.x;
    long row0 = static_cast<long>(blockIdx.x) * blocks_per_wg * 32;
    U4 kf[8], vr[8];
    unsigned acc = 0;
    kv_block<NT>(kf, vr, K, V, row0, lane);
    for (long b = 0; b < blocks_per_wg; ++b) {
        unsigned t = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) t ^= kf[i].x ^ kf[i].w ^ vr[i].y ^ vr[i].z;
        acc += t;
        const long next = b + 1 < blocks_per_wg ? row0 + 32 : row0;
        kv_block<NT>(kf, vr, K, V, next, lane);
        row0 = next;
    }
    out[blockIdx.x * 64 + lane] = acc;
}

void check(hipError_t e, const char* what) {
    if (e != hipSuccess) {
        std::fprintf(stderr, "hbm_read_probe: %s: %s\n", what, hipGetErrorString(e));
        std::exit(1);
    }
}

// Median of `reps` timed launches (after warm-up), in ms.
template <class Launch>
float time_ms(Launch launch, int reps) {
    hipEvent_t e0, e1;
    check(hipEventCreate(&e0), "event");
    check(hipEventCreate(&e1), "event");
    for (int w = 0; w < 3; ++w) launch();
    check(hipDeviceSynchronize(), "warm-up");
    std::vector<float> t;
    for (int r = 0; r < reps; ++r) {
        check(hipEventRecord(e0, nullptr), "record");
        launch();
        check(hipEventRecord(e1, nullptr), "record");
        check(hipEventSynchronize(e1), "sync");
        float ms = 0.f;
        check(hipEventElapsedTime(&ms, e0, e1), "elapsed");
        t.push_back(ms);
    }
    check(hipGetLastError(), "launch");
    std::sort(t.begin(), t.end());
    check(hipEventDestroy(e0), "event");
    check(hipEventDestroy(e1), "event");
    return t[t.size() / 2];
}

}  // namespace

int main() {
    const size_t half = size_t(2) << 30;  // two 2 GiB buffers
    U4 *a = nullptr, *b = nullptr;
    unsigned* out = nullptr;
    constexpr int kMaxGrid = 4096;
    check(hipMalloc(&a, half), "malloc");
    check(hipMalloc(&b, half), "malloc");
    check(hipMalloc(&out, size_t(kMaxGrid) * 64 * sizeof(unsigned)), "malloc");
    check(hipMemset(a, 1, half), "memset");
    check(hipMemset(b, 2, half), "memset");
    int cus = 0;
    check(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0), "attribute");

    // best[nt][kind]: kind 0 = flat, 1 = kv
    double best[2][2] = {{0.0, 0.0}, {0.0, 0.0}};
    int best_grid[2][2] = {{0, 0}, {0, 0}};
    for (int nt = 0; nt < 2; ++nt) {
        // flat: one 2 GiB buffer, one contiguous range per workgroup
        for (int per_cu : {4, 8, 16}) {
            const int grid = std::min(per_cu * cus, kMaxGrid);
            const size_t n16 = half / 16;
            size_t per_wg = n16 / grid / (128 * kFlatU) * (128 * kFlatU);
            if (per_wg < 128 * kFlatU || static_cast<size_t>(grid) * per_wg > n16) continue;
            const float ms = time_ms(
                [&] {
                    if (nt) hipLaunchKernelGGL(flat_read<true>, dim3(grid), dim3(64), 0, nullptr, a, per_wg, out);
                    else hipLaunchKernelGGL(flat_read<false>, dim3(grid), dim3(64), 0, nullptr, a, per_wg, out);
                },
                10);
            const double gbs = static_cast<double>(grid) * per_wg * 16 / (ms * 1e6);
            if (gbs > best[nt][0]) {
                best[nt][0] = gbs;
                best_grid[nt][0] = grid;
            }
        }
        // kv: the attention kernels' access shape over two 2 GiB tensors
        for (int per_cu : {4, 8}) {
            const int grid = std::min(per_cu * cus, kMaxGrid);
            const long rows = static_cast<long>(half / 256);
            const long bpw = rows / 32 / grid;
            if (bpw < 1 || static_cast<long>(grid) * bpw * 32 > rows) continue;
            const float ms = time_ms(
                [&] {
                    if (nt) hipLaunchKernelGGL(kv_read<true>, dim3(grid), dim3(64), 0, nullptr, a, b, bpw, out);
                    else hipLaunchKernelGGL(kv_read<false>, dim3(grid), dim3(64), 0, nullptr, a, b, bpw, out);
                },
                10);
            const double gbs = static_cast<double>(grid) * bpw * 32 * 256 * 2 / (ms * 1e6);
            if (gbs > best[nt][1]) {
                best[nt][1] = gbs;
                best_grid[nt][1] = grid;
            }
        }
    }
    check(hipFree(a), "free");
    check(hipFree(b), "free");
    check(hipFree(out), "free");
    const double kv = std::max(best[0][1], best[1][1]);
    std::printf("{\"flat_read_GBs\": %.1f, \"flat_nt_read_GBs\": %.1f, \"kv_plain_read_GBs\": %.1f, "
                "\"kv_nt_read_GBs\": %.1f, \"kv_read_GBs\": %.1f, \"flat_grid\": %d, \"kv_grid\": %d, \"cus\": %d}\n",
                best[0][0], best[1][0], best[0][1], best[1][1], kv, best_grid[1][0], best_grid[1][1], cus);
    return 0;
}
