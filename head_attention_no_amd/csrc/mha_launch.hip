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

// The current device's compute units and the workgroups of `kernel` (with
// `threads` threads) each one holds at once, cached per device (packed as
// cus * 64 + per_cu); {0, 0} if the runtime cannot tell.
struct Residency {
    int cus, per_cu;
};
Residency residency(const void *kernel, int threads, std::atomic<int> (&cache)[kMaxDevices])
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return {0, 0};
    if (dev < kMaxDevices) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return {c / 64, c % 64};
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
        cus <= 0 || per_cu <= 0 || per_cu >= 64)
        return {0, 0};
    if (dev < kMaxDevices) cache[dev].store(cus * 64 + per_cu, std::memory_order_relaxed);
    return {cus, per_cu};
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
        // D = 64 and 128) launches the resident workgroup count rounded down
        // to a multiple of 8 (the XCDs) when the items outnumber it; each
        // workgroup then walks several items. Where two workgroups fit a
        // compute unit (D = 64) and the items fit the resident count but
        // outnumber the compute units, it launches one workgroup per unit
        // instead: launched all at once, a causal call's items of equal
        // length could share a unit while others idle, where walking pairs
        // each unit's long item with a short one (MHA causal B=4 S=2048 at
        // D = 64: 512 items, 66 against 51 us).
        if constexpr (Tile16<D>::WALK) {
            if (p.walk) {
                static std::atomic<int> cache[2][kMaxDevices];  // per kernel variant
                const Residency r = residency(kernel, threads, cache[p.prescale ? 1 : 0]);
                const int slots = r.cus * r.per_cu / 8 * 8, one = r.cus / 8 * 8;
                if (slots > 0 && slots < n_items)
                    grid = slots;
                else if (r.per_cu > 1 && one > 0 && one < n_items)
                    grid = one;
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
