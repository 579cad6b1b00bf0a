// One (element type, head dim) instance of the attention-forward kernels,
// for all three mask kinds. Compiled once per pair with
// -DFA355_ELEM=<0 float | 1 bf16 | 2 fp16> and -DFA355_HEAD_DIM=<32|64|128|256>.
#include "mha_launch.hpp"

#include <type_traits>

#include "mha_fwd16.hpp"
#include "mha_fwd32.hpp"

#if !defined(FA355_ELEM) || !defined(FA355_HEAD_DIM)
#error "compile with -DFA355_ELEM and -DFA355_HEAD_DIM"
#endif

namespace fa355 {

namespace {

template <typename T, int D, int MASK>
hipError_t launch_one(const Params &p, int grid, hipStream_t stream)
{
    void *args[] = {const_cast<Params *>(&p)};
    if constexpr (std::is_same_v<T, float>)
        return hipLaunchKernel(reinterpret_cast<const void *>(&mha_fwd32<D, MASK>), dim3(grid),
                               dim3(kThreads32), args, 0, stream);
    else
        return hipLaunchKernel(reinterpret_cast<const void *>(&mha_fwd16<T, D, MASK>), dim3(grid),
                               dim3(64 * Tile16<D>::NW), args, 0, stream);
}

}  // namespace

template <typename T, int D>
hipError_t launch_mha(const Params &p, int mask, int grid, hipStream_t stream)
{
    switch (mask) {
    case kMaskNone: return launch_one<T, D, kMaskNone>(p, grid, stream);
    case kMaskCausal: return launch_one<T, D, kMaskCausal>(p, grid, stream);
    default: return launch_one<T, D, kMaskWindow>(p, grid, stream);
    }
}

#if FA355_ELEM == 0
template hipError_t launch_mha<float, FA355_HEAD_DIM>(const Params &, int, int, hipStream_t);
#elif FA355_ELEM == 1
template hipError_t launch_mha<__bf16, FA355_HEAD_DIM>(const Params &, int, int, hipStream_t);
#else
template hipError_t launch_mha<_Float16, FA355_HEAD_DIM>(const Params &, int, int, hipStream_t);
#endif

}  // namespace fa355
