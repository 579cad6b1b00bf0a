// One (element type, head dim) instance of the attention-forward kernels,
// for all three mask kinds. Compiled once per pair with
// -DFA355_ELEM=<0 float | 1 bf16 | 2 fp16> and -DFA355_HEAD_DIM=<32|64|128|256>.
#include "mha_launch.hpp"

#include <atomic>
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

template <typename T, int D, int MASK>
hipError_t launch_one(const Params &p, int n_items, hipStream_t stream)
{
    void *args[] = {const_cast<Params *>(&p)};
    if constexpr (std::is_same_v<T, float>) {
        if constexpr (split_dim32(D)) {
            if (p.kv_split)
                return hipLaunchKernel(reinterpret_cast<const void *>(&mha_fwd32<D, MASK, true>),
                                       dim3(n_items), dim3(kThreads32), args, 0, stream);
        }
        return hipLaunchKernel(reinterpret_cast<const void *>(&mha_fwd32<D, MASK, false>), dim3(n_items),
                               dim3(kThreads32), args, 0, stream);
    } else {
        const void *kernel = reinterpret_cast<const void *>(&mha_fwd16<T, D, MASK, false>);
        int threads = 64 * Tile16<D>::NW;
        if constexpr (Tile16<D>::PRESCALE) {
            if (p.prescale) kernel = reinterpret_cast<const void *>(&mha_fwd16<T, D, MASK, true>);
        }
        if constexpr (D == 256) {
            if (p.few) {
                kernel = reinterpret_cast<const void *>(&mha_fwd16<T, D, MASK, false, true>);
                threads = 64 * Tile16<D, true>::NW;
            }
        }
        int grid = n_items;
        // A walking call (p.walk, set by the C-ABI layer for short items at
        // D = 128) launches the resident workgroup count rounded down to a
        // multiple of 8 (the XCDs) when the items outnumber it; each
        // workgroup then walks several items.
        if constexpr (Tile16<D>::WALK) {
            if (p.walk) {
                static std::atomic<int> cache[2][kMaxDevices];  // per kernel variant
                const int slots = resident_workgroups(kernel, threads, cache[p.prescale ? 1 : 0]) / 8 * 8;
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
