// Shared pieces of the gfx950 attention-forward kernels: kernel arguments,
// the workgroup -> tile map, masks and small device helpers.
//
// The operation is the no-KV-cache attention of the "FlashAttentionGPU" API
// page (max.modular.com, section "execute", Steps 0-4):
// answer = softmax(mask(scale * Q K^T)) V per (batch, head), BSHD in and out,
// K/V heads shared by H/Hkv consecutive query heads (grouped attention).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa355 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

enum MaskKind { kMaskNone = 0, kMaskCausal = 1, kMaskWindow = 2 };

// Kernel arguments (one struct, passed by value).
struct Params {
    void *out;
    const void *q;
    const void *k;
    const void *v;
    int B, S, H, Hkv;
    int rep;       // H / Hkv: query heads per K/V head
    int hp;        // query heads per workgroup: a divisor of rep, so they share one K/V head
    int wph;       // waves per query head: the workgroup's waves / hp
    int n_qtiles;  // ceil(S / query rows per head per workgroup)
    int n_items;   // work items: n_qtiles * B * H / hp (the grid may be smaller)
    int walk;      // 1: a grid below n_items makes each workgroup walk several items
    int group_order;  // 1: items in group order (see block_coord)
    int kv_split;  // 1: fp32 key split (mha_fwd32.hpp): 32-row items, keys split over the waves
    int prescale;  // 1: 16-bit kernel with Q pre-scaled by scale_log2 (mha_fwd16.hpp, D <= 64)
    int few;       // 1: the few-item layout of the 16-bit kernel at D = 256 (Tile16 in mha_fwd16.hpp)
    int window;    // sliding-window width, clamped to S (a window >= S is causal)
    float scale_log2;  // |scale| * log2(e): exp(scale*s) = exp2(s * scale_log2) for scale >= 0
    uint32_t q_sign;   // sign-bit mask XORed into Q so that scale < 0 becomes |scale|
};

// Lazy rescaling: the running max is only raised when a new tile's max
// exceeds it by more than this many powers of two, so P stays <= 2^8 and
// most tiles skip the O rescale altogether.
constexpr float kRescaleLog2 = 8.0f;

// Workgroup -> (query tile, batch, first head h). A workgroup computes the
// same query rows of hp consecutive heads h .. h+hp-1, which share one K/V
// head (hp divides H/Hkv): its waves split as hp heads x (waves / hp) row
// blocks of 32, and all of them read the one K/V tile in LDS. Packing heads
// instead of rows keeps a workgroup's rows few, so under a causal or window
// mask its waves see nearly the same key range and none idles at the
// per-tile barrier while the others work.
// Hardware dispatches workgroup w to XCD w % 8 as that XCD's (w / 8)-th
// workgroup. When the (batch, K/V head) groups split evenly over the 8 XCDs,
// every item of a group runs on one XCD (item w on XCD w % 8), so all the
// query heads that share K/V also share that XCD's L2. Within an XCD, items
// are ordered by slot = w / 8:
//  * launch order (one workgroup per item): longest query tiles (the last
//    ones, under a causal mask) first, across the XCD's groups, so the
//    dispatcher's tail is short;
//  * group order (calls that walk, and unmasked 16-bit calls, whose items
//    are all alike): group by group, each group's query tiles longest
//    first, so the items in flight on an XCD share few K/V heads and their
//    K/V stays in its L2. A walking call takes the items in rounds, forward
//    then back, so a group's long and short tiles land in alternate rounds,
//    which keeps the per-workgroup totals balanced.
// Without an even split, the longest tiles come first.
struct TileCoord {
    int qt, b, h;
};

__host__ __device__ inline TileCoord block_coord(int w, int n_qtiles, int B, int H, int Hkv, int hp,
                                                 int group_order)
{
    const int reps = H / Hkv / hp;  // items per (batch, K/V head) and query tile
    const int groups = B * Hkv;
    TileCoord c;
    if (groups % 8 == 0) {
        const int x = w % 8, slot = w / 8;
        int qi, grp_local, r;
        if (group_order) {
            grp_local = slot / (n_qtiles * reps);
            qi = (slot / reps) % n_qtiles;
            r = slot % reps;
        } else {
            const int per_tile = (groups / 8) * reps;
            qi = slot / per_tile;
            grp_local = (slot % per_tile) / reps;
            r = slot % reps;
        }
        const int grp = grp_local * 8 + x;
        c.b = grp / Hkv;
        c.h = ((grp % Hkv) * reps + r) * hp;
        c.qt = n_qtiles - 1 - qi;
    } else {
        const int hg = H / hp, bh = B * hg;
        c.qt = n_qtiles - 1 - w / bh;
        c.b = (w % bh) / hg;
        c.h = (w % hg) * hp;
    }
    return c;
}

// Key tiles a work item of `rows` query rows visits under mask kind `mask`,
// on average over the query tiles (a close form for the launch heuristic).
inline double mean_key_tiles(int mask, int S, int W, int rows, int BN)
{
    const double all = (S + BN - 1) / BN;
    if (mask == kMaskNone) return all;
    const double seen = mask == kMaskCausal ? S / 2.0 : (W < S / 2.0 ? W : S / 2.0);
    const double m = (seen + rows) / BN;
    return m < all ? m : all;
}

// Whether a call walks its items (walk order, and a resident grid when the
// items outnumber it): the 16-bit kernel at head dim 64 or 128, for items of
// at most 64 key tiles on average. Walking hides each item's start (its Q
// rows and first K/V tile arrive during the previous item's last tile) but
// costs a little per tile. On MI355X at D = 128 it was 6 % faster at window
// 1024, 1.5 % at causal S = 4096 and 1.4 % slower at causal S = 16384; at
// D = 64, 8 %-10 % faster on causal and windowed shapes; at head dim 32,
// which is bound by the vector units, slower at every length.
inline bool walks(bool bits16, int D, int mask, int S, int W, int rows, int BN)
{
    return bits16 && (D == 64 || D == 128) && mean_key_tiles(mask, S, W, rows, BN) <= 64.0;
}

// Tile classification for one wave's 32 rows [r0, r0+31] and keys [k0, k1].
enum TileClass { kEmpty = 0, kFull = 1, kEdge = 2 };

template <int MASK>
__device__ inline int classify(int r0, int k0, int k1, int S, int W)
{
    if (r0 >= S) return kEmpty;  // padding rows only
    const int r1 = r0 + 31;
    const bool tail = k1 >= S;
    if (MASK == kMaskNone) return tail ? kEdge : kFull;
    if (k0 > r1) return kEmpty;
    if (MASK == kMaskWindow && k1 <= r0 - W) return kEmpty;
    bool full = k1 <= r0 && !tail;
    if (MASK == kMaskWindow) full = full && k0 > r1 - W;
    return full ? kFull : kEdge;
}

// The mask functor plus the end of the sequence: may query `row` see `key`?
template <int MASK>
__device__ inline bool visible(int row, int key, int S, int W)
{
    if (key >= S) return false;
    if (MASK == kMaskNone) return true;
    if (key > row) return false;
    if (MASK == kMaskWindow) return key > row - W;
    return true;
}

// The keys query `row` may see among key0 .. key0 + n - 1 (the set visible()
// accepts), as offsets from key0: off in [lo, hi]. Without a window lo is
// not needed (the set starts at key 0); with one, an empty set comes back
// as lo = hi = n, which the test (unsigned)(off - lo) <= hi - lo rejects
// for every off in 0 .. n-1.
template <int MASK>
__device__ inline void visible_range(int row, int key0, int S, int W, int n, int &lo, int &hi)
{
    hi = (MASK == kMaskNone ? S - 1 : min(row, S - 1)) - key0;
    lo = MASK == kMaskWindow ? row - W + 1 - key0 : 0;
    if (MASK == kMaskWindow && hi < lo) lo = hi = n;
}

// Key-tile range [begin, end) a workgroup whose rows (per head) are
// q0 .. q0+rows-1 must visit.
template <int MASK, int BN>
__device__ inline void key_tile_range(int q0, int rows, int S, int W, int &begin, int &end)
{
    const int q_last = min(q0 + rows, S) - 1;
    begin = 0;
    end = (S + BN - 1) / BN;
    if (MASK != kMaskNone) end = min(end, q_last / BN + 1);
    if (MASK == kMaskWindow) begin = max(0, q0 - W + 1) / BN;
}

// ---------------------------------------------------------------------------
// device helpers

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, unrolled at compile time.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_from(F &f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for_from<I + 1, N>(f);
    }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_from<0, N>(f);
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine a per-lane value with the one held by lane ^ 32 (the other half of
// the same query row): returns op(x[lane], x[lane ^ 32]) in every lane.
__device__ inline float half_max(float x)
{
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ inline float half_sum(float x)
{
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ inline bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

// Round 2 floats to a packed pair of 16-bit values (round to nearest even).
template <typename T>
__device__ inline uint32_t pack2(float a, float b);

template <>
__device__ inline uint32_t pack2<__bf16>(float a, float b)
{
    f32x2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

template <>
__device__ inline uint32_t pack2<_Float16>(float a, float b)
{
    f32x2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}

// acc + lo(x) + hi(x) for a packed pair of 16-bit values, in fp32.
template <typename T>
__device__ inline float sum2(uint32_t x, float acc);

template <>
__device__ inline float sum2<__bf16>(uint32_t x, float acc)
{
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), one, acc, false);
}

template <>
__device__ inline float sum2<_Float16>(uint32_t x, float acc)
{
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), one, acc, false);
}

// D = A B + C on a 32x32x16 16-bit MFMA (A: 32 rows x 16 k, B: 16 k x 32 cols).
template <typename T>
__device__ inline f32x16 mfma16(u32x4 a, u32x4 b, f32x16 c);

template <>
__device__ inline f32x16 mfma16<__bf16>(u32x4 a, u32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <>
__device__ inline f32x16 mfma16<_Float16>(u32x4 a, u32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ inline u32x4 ldg16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

}  // namespace fa355
