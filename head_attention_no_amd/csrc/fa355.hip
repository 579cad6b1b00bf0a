// libfa355: C ABI of the fused no-KV-cache attention forward (see fa355.h).
//
// Host side: argument validation (before any HIP call), the gfx950 device
// check, the choice of kernel instance (dtype x head dim x mask kind) and the
// launch on the caller's stream. The attention kernel instances are compiled
// in mha_launch.hip; this unit holds the top-K kernel.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "fa355.h"
#include "mha_fwd16.hpp"
#include "mha_fwd32.hpp"
#include "mha_launch.hpp"
#include "topk.hpp"

namespace {

using fa355::Params;

constexpr double kLog2e = 1.4426950408889634;

const char *const kStatusText[] = {
    "success",
    "invalid argument (null pointer, size < 1, H not a multiple of Hkv, unknown dtype or mask, "
    "window < 1 with the sliding mask, non-finite scale or |scale| * log2(e) beyond the fp32 range, "
    "or out overlapping an input)",
    "unsupported (head dim other than 32, 64, 128 or 256, pointer not 16-byte aligned, grid too large, "
    "or one token row of q over 16 MiB)",
    "no usable device (no current HIP device, or it is not gfx950)",
    "kernel launch failed",
};

int elem_size(int dtype) { return dtype == FA355_F32 ? 4 : 2; }

// Largest token row of q (H * D elements; k and v rows are no longer).
constexpr int64_t kMaxRowBytes = (int64_t)1 << 24;

bool overlaps(const void *a, int64_t na, const void *b, int64_t nb)
{
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

bool supported_dim(int D) { return D == 32 || D == 64 || D == 128 || D == 256; }

// Waves per workgroup of the kernel instance for (dtype, D, few-item
// layout); D must be supported.
int waves_per_wg(int dtype, int D, bool few)
{
    if (dtype == FA355_F32) return fa355::kWaves32;
    switch (D) {
    case 32: return fa355::Tile16<32>::NW;
    case 64: return fa355::Tile16<64>::NW;
    case 128: return fa355::Tile16<128>::NW;
    default: return few ? fa355::Tile16<256, true>::NW : fa355::Tile16<256>::NW;
    }
}
// Query heads per workgroup: the largest of 8, 4, 2, 1 that divides H / Hkv
// and does not exceed the workgroup's waves. Those heads share one K/V head.
int heads_per_wg(int dtype, int D, bool few, int rep)
{
    for (int hp = 8; hp > 1; hp /= 2)
        if (hp <= waves_per_wg(dtype, D, few) && rep % hp == 0) return hp;
    return 1;
}
int block_n(int dtype, int D, bool few)
{
    if (dtype == FA355_F32) return fa355::Tile32<64>::BN;
    switch (D) {
    case 32: return fa355::Tile16<32>::BN;
    case 64: return fa355::Tile16<64>::BN;
    case 128: return fa355::Tile16<128>::BN;
    default: return few ? fa355::Tile16<256, true>::BN : fa355::Tile16<256>::BN;
    }
}

// fp32 calls whose 32-row items number at most this many run the key-split
// instance (mha_fwd32.hpp): one 32-row item per workgroup, its waves taking
// every fourth key tile. Below one item per compute unit the call is bound
// by each wave's serial MFMA chain, which the split shortens fourfold.
constexpr int64_t kSplitMaxItems = 256;

// 16-bit calls at D = 256 whose work items in the default layout (8 waves)
// number fewer than this many per compute unit take the few-item layout
// (4 waves, half the rows per item): 2 under a mask, whose items differ in
// length, and 1 without one. On MI355X (256 compute units) the default
// layout was 6-20 % faster from 512 causal items (256 unmasked) up, and up
// to 1.7x slower below.
constexpr int64_t kComputeUnits = 256;
int64_t few_items_below(int mask_kind) { return (mask_kind == FA355_MASK_NONE ? 1 : 2) * kComputeUnits; }

// How a call is decomposed: heads and rows per workgroup, key tile, items.
struct Layout {
    int hp;     // query heads per workgroup (sharing one K/V head)
    int wph;    // waves per query head
    int bm;     // query rows per head per workgroup
    int bn;     // keys per tile
    int split;  // fp32 key split
    int few;    // the few-item layout at D = 256
    int64_t n_qtiles, n_items;
};

Layout layout_with(int B, int S, int H, int Hkv, int D, int dtype, bool few)
{
    Layout L;
    const int rep = H / Hkv;
    const int64_t items32 = ((int64_t)S + 31) / 32 * B * H;
    L.split = dtype == FA355_F32 && fa355::split_dim32(D) && items32 <= kSplitMaxItems;
    L.few = few ? 1 : 0;
    L.hp = L.split ? 1 : heads_per_wg(dtype, D, few, rep);
    L.wph = L.split ? 1 : waves_per_wg(dtype, D, few) / L.hp;
    L.bm = 32 * L.wph;
    L.bn = block_n(dtype, D, few);
    L.n_qtiles = ((int64_t)S + L.bm - 1) / L.bm;
    L.n_items = L.n_qtiles * B * (H / L.hp);
    return L;
}

// D must be supported and H a multiple of Hkv; mask_kind decides between
// the two layouts at D = 256 (any value is accepted here).
Layout layout_of(int B, int S, int H, int Hkv, int D, int dtype, int mask_kind)
{
    const Layout L = layout_with(B, S, H, Hkv, D, dtype, false);
    if (dtype != FA355_F32 && D == 256 && L.n_items < few_items_below(mask_kind))
        return layout_with(B, S, H, Hkv, D, dtype, true);
    return L;
}

// Shape checks shared by mha_no_cache and fa355_plan.
int check_shape(int B, int S, int H, int Hkv, int D, int dtype)
{
    if (B < 1 || S < 1 || H < 1 || Hkv < 1 || D < 1) return FA355_ERR_INVALID_ARG;
    if (H % Hkv != 0) return FA355_ERR_INVALID_ARG;
    if (dtype != FA355_F32 && dtype != FA355_BF16 && dtype != FA355_F16)
        return FA355_ERR_INVALID_ARG;
    if (!supported_dim(D)) return FA355_ERR_UNSUPPORTED;
    if (layout_with(B, S, H, Hkv, D, dtype, D == 256 && dtype != FA355_F32).n_items > INT32_MAX)
        return FA355_ERR_UNSUPPORTED;  // the layout with the most items
    // Buffer offsets inside one tile are 32-bit: a tile spans at most 128
    // token rows of K/V and 32 of Q, so one token's row of q (H * D
    // elements) or of k / v (Hkv * D elements) may hold at most 16 MiB.
    // Every offset across tokens, heads and batches is 64-bit.
    if ((int64_t)H * D * elem_size(dtype) > kMaxRowBytes) return FA355_ERR_UNSUPPORTED;
    return FA355_OK;
}

// Mask kind and window as mha_no_cache checks them.
int check_mask(int mask_kind, int window)
{
    if (mask_kind != FA355_MASK_NONE && mask_kind != FA355_MASK_CAUSAL &&
        mask_kind != FA355_MASK_SLIDING_WINDOW)
        return FA355_ERR_INVALID_ARG;
    if (mask_kind == FA355_MASK_SLIDING_WINDOW && window < 1) return FA355_ERR_INVALID_ARG;
    return FA355_OK;
}

// Window width the kernels use: clamped to S (a window >= S is causal).
int clamped_window(int mask_kind, int window, int S)
{
    return mask_kind == FA355_MASK_SLIDING_WINDOW ? (window < S ? window : S) : S;
}

// Whether the call walks its work items (see fa355::walks).
int call_walks(int dtype, int D, const Layout &L, int mask_kind, int S, int window_clamped)
{
    return fa355::walks(dtype != FA355_F32, D, mask_kind, S, window_clamped, L.bm, L.bn) ? 1 : 0;
}

// Whether the items are ordered group by group (see fa355::block_coord):
// calls that walk, and unmasked 16-bit calls (all their items are alike, so
// nothing is gained by running the longest first, and group order keeps the
// K/V of the items in flight on an XCD within its L2).
int call_group_order(int dtype, int mask_kind, int walk)
{
    return walk || (dtype != FA355_F32 && mask_kind == FA355_MASK_NONE) ? 1 : 0;
}

// Per-device cache of the architecture check: 0 unknown, 1 gfx950, 2 other.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];

int check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA355_ERR_DEVICE;
    int state = dev < kMaxDevices ? g_arch_state[dev].load(std::memory_order_relaxed) : 0;
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FA355_ERR_DEVICE;
        state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (dev < kMaxDevices) g_arch_state[dev].store(state, std::memory_order_relaxed);
    }
    return state == 1 ? FA355_OK : FA355_ERR_DEVICE;
}

template <typename T>
hipError_t launch_dim(const Params &p, int D, int mask, hipStream_t stream)
{
    switch (D) {
    case 32: return fa355::launch_mha<T, 32>(p, mask, stream);
    case 64: return fa355::launch_mha<T, 64>(p, mask, stream);
    case 128: return fa355::launch_mha<T, 128>(p, mask, stream);
    default: return fa355::launch_mha<T, 256>(p, mask, stream);
    }
}

}  // namespace

extern "C" int mha_no_cache(void *out, const void *q, const void *k, const void *v, int B, int S,
                            int H, int Hkv, int D, float scale, int mask_kind, int window,
                            int dtype, void *stream)
{
    // Validation: no HIP call before every argument has been checked.
    if (!out || !q || !k || !v) return FA355_ERR_INVALID_ARG;
    int rc = check_shape(B, S, H, Hkv, D, dtype);
    if (rc == FA355_ERR_INVALID_ARG) return rc;
    if (check_mask(mask_kind, window) != FA355_OK) return FA355_ERR_INVALID_ARG;
    // |scale| * log2(e) is the kernels' fp32 exponent scale: it must be finite.
    if (!std::isfinite(scale) || std::fabs((double)scale) * kLog2e > (double)FLT_MAX)
        return FA355_ERR_INVALID_ARG;
    const int64_t es = elem_size(dtype);
    const int64_t q_bytes = (int64_t)B * S * H * D * es;
    const int64_t kv_bytes = (int64_t)B * S * Hkv * D * es;
    if (overlaps(out, q_bytes, q, q_bytes) || overlaps(out, q_bytes, k, kv_bytes) ||
        overlaps(out, q_bytes, v, kv_bytes))
        return FA355_ERR_INVALID_ARG;
    if (rc != FA355_OK) return rc;
    if (((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(q) |
          reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) &
         15u) != 0)
        return FA355_ERR_UNSUPPORTED;

    rc = check_device();
    if (rc != FA355_OK) return rc;

    Params p{};
    p.out = out;
    p.q = q;
    p.k = k;
    p.v = v;
    p.B = B;
    p.S = S;
    p.H = H;
    p.Hkv = Hkv;
    const Layout L = layout_of(B, S, H, Hkv, D, dtype, mask_kind);
    p.rep = H / Hkv;
    p.hp = L.hp;
    p.wph = L.wph;
    p.kv_split = L.split;
    p.few = L.few;
    p.n_qtiles = (int)L.n_qtiles;
    p.window = clamped_window(mask_kind, window, S);
    // exp(scale * s) = exp2(|scale| * log2(e) * (sign(scale) * s)); the sign
    // goes into Q (an exact bit flip) so the kernel's scale is never negative.
    // A scale below 1e-30 in magnitude is taken as 1e-30: for any fp32 score
    // |s| < 1e20 the exponent then stays below 1e-10 and exp2 rounds to
    // exactly 1, as with scale 0, while hidden scores (-inf) still give 0.
    p.scale_log2 = (float)std::fmax(std::fabs((double)scale) * kLog2e, 1e-30);
    const bool neg = std::signbit(scale) && scale != 0.0f;
    p.q_sign = neg ? (dtype == FA355_F32 ? 0x80000000u : 0x80008000u) : 0u;
    // Pre-scaled Q at head dims 32 and 64 (mha_fwd16.hpp), unless the scaled
    // fp16 values could overflow: |q * scale * log2(e)| <= |q| needs
    // |scale| log2(e) <= 1.
    p.prescale = dtype != FA355_F32 && D <= 64 && (dtype == FA355_BF16 || p.scale_log2 <= 1.0f);

    p.n_items = (int)L.n_items;
    p.walk = call_walks(dtype, D, L, mask_kind, S, p.window);
    p.group_order = call_group_order(dtype, mask_kind, p.walk);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    switch (dtype) {
    case FA355_BF16: err = launch_dim<__bf16>(p, D, mask_kind, s); break;
    case FA355_F16: err = launch_dim<_Float16>(p, D, mask_kind, s); break;
    default: err = launch_dim<float>(p, D, mask_kind, s); break;
    }
    return err == hipSuccess ? FA355_OK : FA355_ERR_LAUNCH;
}

extern "C" int fa355_topk(float *values, int *indices, const float *in, int B, int V, int K,
                          void *stream)
{
    if (!values || !indices || !in) return FA355_ERR_INVALID_ARG;
    if (B < 1 || V < 1 || K < 1 || K > V) return FA355_ERR_INVALID_ARG;
    const int64_t in_bytes = (int64_t)B * V * 4, out_bytes = (int64_t)B * K * 4;
    if (overlaps(values, out_bytes, in, in_bytes) || overlaps(indices, out_bytes, in, in_bytes) ||
        overlaps(values, out_bytes, indices, out_bytes))
        return FA355_ERR_INVALID_ARG;
    if (K > fa355::kTopkMaxK) return FA355_ERR_UNSUPPORTED;
    if (((reinterpret_cast<uintptr_t>(values) | reinterpret_cast<uintptr_t>(indices) |
          reinterpret_cast<uintptr_t>(in)) &
         3u) != 0)
        return FA355_ERR_UNSUPPORTED;
    const int rc = check_device();
    if (rc != FA355_OK) return rc;
    fa355::TopkParams p;
    p.values = values;
    p.indices = indices;
    p.in = in;
    p.V = V;
    p.K = K;
    void *args[] = {&p};
    const hipError_t err = hipLaunchKernel(reinterpret_cast<const void *>(&fa355::topk_rows), dim3(B),
                                          dim3(fa355::kTopkThreads), args, 0,
                                          static_cast<hipStream_t>(stream));
    return err == hipSuccess ? FA355_OK : FA355_ERR_LAUNCH;
}

extern "C" const char *fa355_strerror(int status)
{
    if (status < 0 || status > FA355_ERR_LAUNCH) return "unknown status";
    return kStatusText[status];
}

extern "C" const char *fa355_version(void) { return "fa355 0.1.0 gfx950"; }

extern "C" int fa355_plan(int B, int S, int H, int Hkv, int D, int dtype, int mask_kind, int window,
                          int *num_workgroups, int *block_m_out, int *block_n_out,
                          int *heads_per_wg_out, int *walk_out, int *tiles, int n)
{
    int rc = check_shape(B, S, H, Hkv, D, dtype);
    if (rc == FA355_ERR_INVALID_ARG) return rc;
    if (check_mask(mask_kind, window) != FA355_OK) return FA355_ERR_INVALID_ARG;
    if (rc != FA355_OK) return rc;
    const Layout L = layout_of(B, S, H, Hkv, D, dtype, mask_kind);
    const int hp = L.hp, n_qtiles = (int)L.n_qtiles, grid = (int)L.n_items;
    const int walk = call_walks(dtype, D, L, mask_kind, S, clamped_window(mask_kind, window, S));
    if (num_workgroups) *num_workgroups = grid;
    if (block_m_out) *block_m_out = L.bm;
    if (block_n_out) *block_n_out = L.bn;
    if (heads_per_wg_out) *heads_per_wg_out = hp;
    if (walk_out) *walk_out = walk;
    if (tiles) {
        if (n < 0) return FA355_ERR_INVALID_ARG;
        for (int w = 0; w < n && w < grid; ++w) {
            const fa355::TileCoord c =
                fa355::block_coord(w, n_qtiles, B, H, Hkv, hp, call_group_order(dtype, mask_kind, walk));
            tiles[3 * w + 0] = c.qt;
            tiles[3 * w + 1] = c.b;
            tiles[3 * w + 2] = c.h;
        }
    }
    return FA355_OK;
}
