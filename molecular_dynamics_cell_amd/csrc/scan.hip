// Exclusive prefix sum (int32 counts -> int64 offsets) used to turn per-row counts into CSR
// offsets: reduce per block, scan the block totals (recursively), then scan inside blocks.
#include "impl.h"

namespace mpnn {

namespace {

constexpr int kScanThreads = 256;
constexpr int kScanItems = 16;
constexpr int kScanTile = kScanThreads * kScanItems;

template <class TIn>
__global__ void k_tile_sums(const TIn *__restrict__ in, int64_t n, int64_t *__restrict__ sums) {
    __shared__ int64_t sh[kScanThreads];
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
    int64_t s = 0;
    for (int k = 0; k < kScanItems; ++k) {
        int64_t i = base + (int64_t)k * kScanThreads + threadIdx.x;
        if (i < n) s += (int64_t)in[i];
    }
    sh[threadIdx.x] = s;
    __syncthreads();
    for (int w = kScanThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) sums[blockIdx.x] = sh[0];
}

// Scans one tile: thread t owns items [t*kScanItems, (t+1)*kScanItems) of the tile.
template <class TIn>
__global__ void k_tile_scan(const TIn *__restrict__ in, int64_t n, const int64_t *__restrict__ tile_off,
                            int64_t *__restrict__ out, int write_total) {
    __shared__ int64_t sh[kScanThreads];
    const int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanItems;
    int64_t v[kScanItems];
    int64_t s = 0;
    for (int k = 0; k < kScanItems; ++k) {
        int64_t i = base + k;
        v[k] = (i < n) ? (int64_t)in[i] : 0;
        s += v[k];
    }
    sh[threadIdx.x] = s;
    __syncthreads();
    // Hillis-Steele inclusive scan of the per-thread totals
    for (int w = 1; w < kScanThreads; w <<= 1) {
        int64_t add = ((int)threadIdx.x >= w) ? sh[threadIdx.x - w] : 0;
        __syncthreads();
        sh[threadIdx.x] += add;
        __syncthreads();
    }
    int64_t run = (tile_off ? tile_off[blockIdx.x] : 0) + sh[threadIdx.x] - s;
    for (int k = 0; k < kScanItems; ++k) {
        int64_t i = base + k;
        if (i < n) out[i] = run;
        run += v[k];
        if (write_total && i == n - 1) out[n] = run;
    }
}

template <class TIn>
Status scan_impl(Context &cx, const TIn *in, int64_t n, int64_t *out, int64_t *scratch) {
    if (n <= 0) {
        MPNN_HIP(hipMemsetAsync(out, 0, sizeof(int64_t), cx.stream));
        return Status::ok();
    }
    const int64_t tiles = (n + kScanTile - 1) / kScanTile;
    if (tiles == 1) {
        k_tile_scan<TIn><<<1, kScanThreads, 0, cx.stream>>>(in, n, nullptr, out, 1);
        MPNN_HIP(hipGetLastError());
        return Status::ok();
    }
    int64_t *sums = scratch;
    int64_t *offs = scratch + tiles + 1;
    k_tile_sums<TIn><<<(unsigned)tiles, kScanThreads, 0, cx.stream>>>(in, n, sums);
    MPNN_HIP(hipGetLastError());
    MPNN_TRY(scan_impl<int64_t>(cx, sums, tiles, offs, scratch + 2 * (tiles + 1)));
    k_tile_scan<TIn><<<(unsigned)tiles, kScanThreads, 0, cx.stream>>>(in, n, offs, out, 1);
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

// int64 words of scratch needed by scan_impl for n items
int64_t scan_scratch_words(int64_t n) {
    int64_t words = 0;
    while (n > kScanTile) {
        int64_t tiles = (n + kScanTile - 1) / kScanTile;
        words += 2 * (tiles + 1);
        n = tiles;
    }
    return words + 2;
}

}  // namespace

Status exclusive_scan(Context &cx, const int32_t *in, int64_t n, int64_t *out) {
    MPNN_TRY(cx.grow(cx.tmp_scan, sizeof(int64_t) * (size_t)scan_scratch_words(n)));
    return scan_impl<int32_t>(cx, in, n, out, cx.tmp_scan.as<int64_t>());
}

}  // namespace mpnn
