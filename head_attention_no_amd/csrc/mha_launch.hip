// One (element type, head dim) instance of the attention-forward kernels,
// for all three mask kinds. Compiled once per pair with
// -DFA355_ELEM=<0 float | 1 bf16 | 2 fp16> and -DFA355_HEAD_DIM=<32|64|128|256>.
#include "mha_launch.hpp"

#include <atomic>
#include <cmath>
#include <type_traits>

#include "mha_fwd16.hpp"
#include "mha_fwd32.hpp"

#if !defined(FA355_ELEM) || !defined(FA355_HEAD_DIM)
#error "compile with -DFA355_ELEM and -DFA355_HEAD_DIM"
#endif

namespace fa355 {

namespace {

constexpr int kMaxDevices = 64;

// Workgroups of `kernel` (with `threads` threads) the current device holds
// at once: compute units x resident workgroups per unit, cached per device;
// 0 if the runtime cannot tell.
int resident_workgroups(const void *kernel, int threads, std::atomic<int> (&cache)[kMaxDevices])
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDevices) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
        return 0;
    const int n = cus > 0 && per_cu > 0 ? cus * per_cu : 0;
    if (dev < kMaxDevices && n > 0) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Key tiles a work item of `rows` query rows visits, on average over the
// query tiles (close form; only a launch heuristic uses it).
template <int MASK>
double mean_key_tiles(int S, int W, int rows, int BN)
{
    const double all = (S + BN - 1) / BN;
    if (MASK == kMaskNone) return all;
    const double seen = MASK == kMaskCausal ? S / 2.0 : std::fmin((double)W, S / 2.0);
    return std::fmin(all, (seen + rows) / BN);
}

template <typename T, int D, int MASK>
hipError_t launch_one(const Params &p, int n_items, hipStream_t stream)
{
    void *args[] = {const_cast<Params *>(&p)};
    if constexpr (std::is_same_v<T, float>) {
        return hipLaunchKernel(reinterpret_cast<const void *>(&mha_fwd32<D, MASK>), dim3(n_items),
                               dim3(kThreads32), args, 0, stream);
    } else {
        const void *kernel = reinterpret_cast<const void *>(&mha_fwd16<T, D, MASK>);
        constexpr int threads = 64 * Tile16<D>::NW;
        int grid = n_items;
        // The plain-loop kernel can walk several work items per workgroup:
        // the grid is then the resident workgroup count rounded down to a
        // multiple of 8 (the XCDs). Walking hides each item's start (its Q
        // rows and first K/V tile arrive during the previous item's last
        // tile) but costs a little per tile, so it is used where items are
        // short: at D = 128, items of at most 64 key tiles on average (MI355X:
        // 6 % faster at window 1024, 1.5 % at causal S = 4096, 1.4 % slower
        // at causal S = 16384). At D = 32, bound by the vector units, it
        // was slower at every length measured.
        if constexpr (Tile16<D>::WALK) {
            if (mean_key_tiles<MASK>(p.S, p.window, 32 * p.wph, Tile16<D>::BN) <= 64.0) {
                static std::atomic<int> cache[kMaxDevices];
                const int slots = resident_workgroups(kernel, threads, cache) / 8 * 8;
                if (slots > 0 && slots < n_items) grid = slots;
            }
        }
        return hipLaunchKernel(kernel, dim3(grid), dim3(threads), args, 0, stream);
    }
}

}  // namespace

template <typename T, int D>
hipError_t launch_mha(const Params &p, int mask, hipStream_t stream)
{
    switch (mask) {
    case kMaskNone: return launch_one<T, D, kMaskNone>(p, p.n_items, stream);
    case kMaskCausal: return launch_one<T, D, kMaskCausal>(p, p.n_items, stream);
    default: return launch_one<T, D, kMaskWindow>(p, p.n_items, stream);
    }
}

#if FA355_ELEM == 0
template hipError_t launch_mha<float, FA355_HEAD_DIM>(const Params &, int, hipStream_t);
#elif FA355_ELEM == 1
template hipError_t launch_mha<__bf16, FA355_HEAD_DIM>(const Params &, int, hipStream_t);
#else
template hipError_t launch_mha<_Float16, FA355_HEAD_DIM>(const Params &, int, hipStream_t);
#endif

}  // namespace fa355
