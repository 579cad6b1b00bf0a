// Top-K ordering of batch rows for gfx950: the top-K token sampler of the
// recipe page "Custom Operations: Applications in AI Models", section
// "Optimizing top-K token sampling for GPUs in MAX" (each batch row of
// next-word frequencies is ordered by highest frequency; one GPU block per
// row). Result per row: the K largest entries in descending order, equal
// values by ascending index (-0.0 equals +0.0), as values and indices.
//
// One 1024-thread workgroup (16 waves) per row. Floats map to unsigned
// order keys (larger float, larger key).
//
// K <= 64 on rows of 16384 entries or more (the sampler's case): one
// read. Up to four full batches of 16384 entries stream in; each thread's
// largest entry among them bounds the row's K-th largest from below (their K-th largest, found with a histogram of
// the top 12 key bits), and the rest of the row streams while every entry
// at or above the bound joins a candidate list in LDS. Up to 256
// candidates are ranked by counting (all waves share the comparisons);
// more are sorted in 64-entry chunks in registers (bitonic network over
// DPP and permlane exchanges) and merged by a tree of bitonic merges. A
// list of more than 5120 candidates (heavily tied rows) sends the row to
// the paths below.
//
// Otherwise, long rows first try one read: a histogram of the first 8192
// entries bounds the K-th largest key from below, and the one read keeps
// every entry above the bound as a candidate in LDS unless there are more
// than 4096. Otherwise a histogram of the top 12 key bits (in LDS) finds
// the bin of the K-th largest entry of the row. Usually that bin holds few
// entries: a second and last read of the row then collects the entries of
// higher bins and those of the bin itself (candidates, at most 4096) into
// LDS, where a radix select over the candidates picks the ones still
// needed. When the bin is larger, the radix select continues over the
// next 12 and 8 bits (stopping once every entry sharing the prefix is
// wanted), and a gather pass takes the entries above the prefix and the
// tied entries in index order (block-wide prefix counts over each chunk of
// the row). Either way a last bitonic sort of the K chosen (key, index)
// pairs orders them.
#pragma once

#include "mha_common.hpp"

namespace fa355 {

constexpr int kTopkThreads = 1024;
constexpr int kTopkMaxK = 1024;
constexpr int kTopkUnroll = 4;  // float4 loads in flight per thread and chunk
constexpr int kTopkCand = 4096;  // LDS room for the entries of the threshold bin
constexpr int kTopkChunkVec = 2048;  // float4 vectors in the first chunk (8192 entries)
constexpr int kTopkSmallK = 64;      // the wave-sort path: K up to one wave's lanes
constexpr int kTopkBatchVec = kTopkThreads * kTopkUnroll;  // float4 vectors per batch (16384 entries)
constexpr int kTopkListCap = 5120;   // candidate slots on the wave-sort path
constexpr int kTopkRankMax = 256;    // up to this many candidates, selection by rank

// LDS beside the 4096-bin histogram: either the selection and candidate
// arrays of the paths that read the row twice, or the wave-sort path's
// candidate list.
union TopkLds {
    struct {
        uint32_t sel_key[kTopkMaxK];
        int32_t sel_idx[kTopkMaxK];
        uint32_t cand_key[kTopkCand];
        int32_t cand_idx[kTopkCand];
    } g;
    uint64_t list[kTopkListCap];
};
static_assert(sizeof(uint64_t[kTopkListCap]) <= 2 * kTopkMaxK * 4 + 2 * kTopkCand * 4,
              "the list shares the selection arrays' space");

struct TopkParams {
    float *values;
    int32_t *indices;
    const float *in;
    int V, K;
};

// Order key: unsigned compare of keys = float compare of values; -0.0 and
// +0.0 get the same key.
__device__ inline uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave-sort path entries: 64-bit words whose unsigned order is the result
// order. High word: the order key; low word: (0x7FFFFFFF - index) << 1,
// larger for lower indices, with bit 0 set for -0.0 (so the value comes
// back bit for bit). 0 sorts after every entry and pads.
__device__ inline uint64_t entry_word(uint32_t bits, int idx)
{
    return ((uint64_t)order_key(__uint_as_float(bits)) << 32) |
           ((uint32_t)(0x7FFFFFFF - idx) << 1) | (uint32_t)(bits == 0x80000000u);
}

__device__ inline int entry_index(uint64_t w) { return 0x7FFFFFFF - (int)((uint32_t)w >> 1); }

__device__ inline float entry_value(uint64_t w)
{
    const uint32_t key = (uint32_t)(w >> 32);
    uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
    if (w & 1u) u = 0x80000000u;
    return __uint_as_float(u);
}

// The value of lane (lane ^ STRIDE), on the vector ALU only. DPP inside
// 16-lane rows: quad permutes for 1 and 2; row rotations for 4 (lane i
// reads lane i - n, n = 4 or 12, by bit 2 of the lane) and 8 (symmetric).
// Across rows: v_permlane16_swap / v_permlane32_swap with the value as
// both operands; the first result then holds, in the upper row (half) of
// each pair, the lower one's values, the second result the converse.
template <int STRIDE>
__device__ inline uint32_t lane_xor(uint32_t v)
{
    const int lane = threadIdx.x & 63;
    if constexpr (STRIDE == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
    } else if constexpr (STRIDE == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
    } else if constexpr (STRIDE == 4) {
        const uint32_t down = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false);  // row_ror:4
        const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x12C, 0xF, 0xF, false);    // row_ror:12
        return (lane & 4) ? down : up;
    } else if constexpr (STRIDE == 8) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
    } else if constexpr (STRIDE == 16) {
        const auto s = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? s[0] : s[1];
    } else {
        const auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane & 32) ? s[0] : s[1];
    }
}

// One compare-exchange of a bitonic network held in a wave, one 64-bit
// entry per lane (as two words): the lane keeps the larger or the smaller
// of its entry and its partner's.
template <int STRIDE>
__device__ inline void wave_cx(uint32_t &hi, uint32_t &lo, bool keep_larger)
{
    const uint32_t ph = lane_xor<STRIDE>(hi), pl = lane_xor<STRIDE>(lo);
    const uint64_t a = ((uint64_t)hi << 32) | lo, b = ((uint64_t)ph << 32) | pl;
    // Equal entries (padding only) may swap: harmless. Selects, no branches.
    const bool take = (b > a) == keep_larger;
    hi = take ? ph : hi;
    lo = take ? pl : lo;
}

// Bitonic merge: a bitonic sequence over the wave's 64 lanes, sorted
// descending (lane 0 largest).
template <int STRIDE>
__device__ inline void wave_merge_desc(uint32_t &hi, uint32_t &lo)
{
    wave_cx<STRIDE>(hi, lo, ((threadIdx.x & 63) & STRIDE) == 0);
    if constexpr (STRIDE > 1) wave_merge_desc<STRIDE / 2>(hi, lo);
}

// Bitonic sort of the wave's 64 entries, descending: blocks of SIZE
// alternate direction until the last, which runs descending.
template <int SIZE, int STRIDE>
__device__ inline void wave_sort_stage(uint32_t &hi, uint32_t &lo)
{
    const int lane = threadIdx.x & 63;
    const bool desc = SIZE == 64 || (lane & SIZE) == 0;
    wave_cx<STRIDE>(hi, lo, ((lane & STRIDE) == 0) == desc);
    if constexpr (STRIDE > 1) wave_sort_stage<SIZE, STRIDE / 2>(hi, lo);
}

template <int SIZE = 2>
__device__ inline void wave_sort_desc(uint32_t &hi, uint32_t &lo)
{
    wave_sort_stage<SIZE, SIZE / 2>(hi, lo);
    if constexpr (SIZE < 64) wave_sort_desc<SIZE * 2>(hi, lo);
}

// Both lists sorted descending; afterwards (hi, lo) holds the 64 largest
// of the two, sorted descending. (rh, rl) is the other list read in
// reverse lane order: the lane-wise larger of a descending and an
// ascending list is a bitonic sequence holding the top half.
__device__ inline void wave_keep_top(uint32_t &hi, uint32_t &lo, uint32_t rh, uint32_t rl)
{
    const uint64_t a = ((uint64_t)hi << 32) | lo, b = ((uint64_t)rh << 32) | rl;
    const bool take = b > a;
    hi = take ? rh : hi;
    lo = take ? rl : lo;
    wave_merge_desc<32>(hi, lo);
}

// Exclusive prefix sum of v over the workgroup in thread order; `total`
// gets the sum over all threads. Uses `scratch` (16 ints of LDS) and two
// barriers, so every thread must call it.
__device__ inline int block_exclusive_sum(int v, int *scratch, int &total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) scratch[wave] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kTopkThreads / 64; ++w) {
        const int s = scratch[w];
        before += (w < wave) ? s : 0;
        tot += s;
    }
    __syncthreads();  // scratch may be reused right after
    total = tot;
    return before + x - v;
}

// One compare-exchange of a bitonic network over (key, index) pairs in LDS:
// pair p of the stage with this stride, in a block of `size` that sorts
// forward (key descending, then index ascending) when bit `size` of the
// lower element is clear.
__device__ inline void bitonic_step(uint32_t *key, int32_t *idx, int p, int stride, int size)
{
    const int i = ((p & ~(stride - 1)) << 1) | (p & (stride - 1));
    const int j = i | stride;
    const uint32_t ki = key[i], kj = key[j];
    const int ii = idx[i], ij = idx[j];
    const bool i_first = ki > kj || (ki == kj && ii < ij);  // i precedes j
    const bool forward = (i & size) == 0;
    if (i_first != forward) {
        key[i] = kj;
        key[j] = ki;
        idx[i] = ij;
        idx[j] = ii;
    }
}

// Sort n (a power of two, <= 4096) (key, index) pairs in LDS by key
// descending, then index ascending; every thread must call it. Up to 128
// elements, one wave sorts them alone, one pair per lane and stage (a
// wave's LDS accesses complete in order, so no barrier is needed between
// stages). Above that, wave w owns elements [w n/16, (w+1) n/16): stages
// whose stride stays inside that slice run per wave without a barrier, and
// only the few wider stages synchronise the workgroup.
__device__ inline void lds_bitonic_sort(uint32_t *key, int32_t *idx, int n)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int npairs = n >> 1;
    if (n <= 128) {
        if (wave == 0)
            for (int size = 2; size <= n; size <<= 1)
                for (int stride = size >> 1; stride > 0; stride >>= 1) {
                    for (int p = lane; p < npairs; p += 64) bitonic_step(key, idx, p, stride, size);
                    __builtin_amdgcn_wave_barrier();
                }
        __syncthreads();
        return;
    }
    const int slice = n / (kTopkThreads / 64);      // elements per wave
    const int wave_pairs = slice >> 1;
    for (int size = 2; size <= n; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= slice) {
                __syncthreads();
                for (int p = threadIdx.x; p < npairs; p += kTopkThreads) bitonic_step(key, idx, p, stride, size);
                __syncthreads();
            } else {
                for (int p = wave * wave_pairs + lane; p < (wave + 1) * wave_pairs; p += 64)
                    bitonic_step(key, idx, p, stride, size);
                __builtin_amdgcn_wave_barrier();
            }
        }
    __syncthreads();
}

// Candidate list of the wave-sort path, and its length.
static __shared__ TopkLds lds;
static __shared__ int list_len;

// Appends the entries among w[0..3] (indices e .. e + 3) that are at or
// above the bound and lie before `end` to the candidate list: one LDS
// atomic per element position that any lane has, ballot compaction inside
// the wave. Every lane of the wave calls it.
__device__ __forceinline__ void topk_append4(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, int e, int end,
                                          bool positive, int lo_bits, uint32_t not_lo)
{
    const int lane = threadIdx.x & 63;
    const uint32_t w[4] = {w0, w1, w2, w3};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const bool cand = e + c < end && (positive ? (int)w[c] >= lo_bits : w[c] <= not_lo);
        const uint64_t m = __builtin_amdgcn_ballot_w64(cand);
        if (m) {
            int base = 0;
            if (lane == 0) base = atomicAdd(&list_len, (int)__builtin_popcountll(m));
            base = __builtin_amdgcn_readfirstlane(base);
            const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (cand && pos < kTopkListCap) lds.list[pos] = entry_word(w[c], e + c);
        }
    }
}

__global__ __launch_bounds__(kTopkThreads) void topk_rows(TopkParams p)
{
    __shared__ __attribute__((aligned(16))) uint32_t hist[4096];
    __shared__ int n_cand, n_tie;
    __shared__ uint32_t top_key;
    __shared__ int scratch[kTopkThreads / 64];
    __shared__ int found[2];  // bin, entries still needed within it
    __shared__ int n_greater;

    const int tid = threadIdx.x;
    const int V = p.V, K = p.K;
    const float *x = p.in + (int64_t)blockIdx.x * V;

    // The row as an aligned float4 body between a scalar head and tail.
    const int head = min(V, (int)(((16u - ((uint32_t)(uintptr_t)x & 15u)) & 15u) >> 2));
    const int nvec = (V - head) >> 2;
    const int tail0 = head + 4 * nvec;
    const float4 *xv = reinterpret_cast<const float4 *>(x + head);

    // Visit every entry (any order): fn(key, index).
    auto for_each = [&](auto &&fn) {
        if (tid < head) fn(order_key(x[tid]), tid);
        for (int i0 = 0; i0 < nvec; i0 += kTopkThreads * kTopkUnroll) {
            float4 v[kTopkUnroll];
#pragma unroll
            for (int u = 0; u < kTopkUnroll; ++u) {
                const int j = i0 + u * kTopkThreads + tid;
                v[u] = j < nvec ? xv[j] : float4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int u = 0; u < kTopkUnroll; ++u) {
                const int j = i0 + u * kTopkThreads + tid;
                if (j < nvec) {
                    const int e = head + 4 * j;
                    fn(order_key(v[u].x), e);
                    fn(order_key(v[u].y), e + 1);
                    fn(order_key(v[u].z), e + 2);
                    fn(order_key(v[u].w), e + 3);
                }
            }
        }
        if (tail0 + tid < V) fn(order_key(x[tail0 + tid]), tail0 + tid);
    };

    // Radix select. Invariant: the wanted entries are all with
    // (key & mask) > prefix, plus `need` of those with (key & mask) == prefix.
    uint32_t prefix = 0u, mask = 0u;
    int need = K;
    constexpr int kShift[3] = {20, 8, 0};
    constexpr int kBits[3] = {12, 12, 8};
    // In hist[0 .. nb), the bin holding the want-th largest counted entry:
    // found[0] = that bin, found[1] = how many of its entries are wanted.
    // Thread t owns bins top, top-1, .. (descending); the prefix sum in
    // thread order counts the entries in higher bins.
    auto find_bin = [&](int nb, int want) {
        const int bpt = nb >= kTopkThreads ? nb / kTopkThreads : 1;
        const int top = nb - 1 - tid * bpt;
        int local = 0;
        for (int b = 0; b < bpt; ++b)
            if (top - b >= 0) local += (int)hist[top - b];
        int total;
        int above = block_exclusive_sum(local, scratch, total);
        for (int b = 0; b < bpt; ++b) {
            if (top - b < 0) break;
            const int c = (int)hist[top - b];
            if (above < want && want <= above + c) {
                found[0] = top - b;
                found[1] = want - above;
            }
            above += c;
        }
        __syncthreads();
    };
    // One digit over the entries `visit` enumerates (fn(key, index) for
    // each); returns how many of them share the new prefix.
    auto radix_pass = [&](int pass, auto &&visit) {
        const int shift = kShift[pass], nb = 1 << kBits[pass];
        for (int i = tid; i < nb; i += kTopkThreads) hist[i] = 0u;
        __syncthreads();
        visit([&](uint32_t key, int) {
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & (nb - 1)], 1u);
        });
        __syncthreads();
        find_bin(nb, need);
        const int bin = found[0];
        const int in_bin = (int)hist[bin];
        prefix |= (uint32_t)bin << shift;
        mask |= (uint32_t)(nb - 1) << shift;
        need = found[1];
        __syncthreads();  // hist and found are rewritten next
        return in_bin;
    };
    auto visit_row = [&](auto &&fn) { for_each(fn); };

    // From the nc candidates in cand_key/cand_idx, the `want` largest (key
    // descending, index ascending) go to sel[base .. base + want), in any
    // order: a radix select over the candidates in LDS, then, if the last
    // digit still ties, the lowest indices of the tied entries.
    auto pick = [&](int nc, int base, int want) {
        auto visit_cand = [&](auto &&fn) {
            for (int i = tid; i < nc; i += kTopkThreads) fn(lds.g.cand_key[i], (int)lds.g.cand_idx[i]);
        };
        prefix = 0u;
        mask = 0u;
        need = want;
        int last = 0;
        for (int pass = 0; pass < 3; ++pass) {
            last = radix_pass(pass, visit_cand);
            if (last == need) break;  // every candidate sharing the prefix is wanted
        }
        const bool by_index = last != need;  // ties at the full key: lowest indices first
        const int gt = want - need;
        if (tid == 0) {
            n_greater = 0;
            n_tie = 0;
        }
        __syncthreads();
        int32_t *tie = reinterpret_cast<int32_t *>(hist);
        visit_cand([&](uint32_t key, int idx) {
            const uint32_t k = key & mask;
            if (k > prefix) {
                const int s = atomicAdd(&n_greater, 1);  // < gt by the select invariant
                if (s < gt) {
                    lds.g.sel_key[base + s] = key;
                    lds.g.sel_idx[base + s] = idx;
                }
            } else if (k == prefix) {
                const int s = atomicAdd(&n_tie, 1);  // < last
                if (!by_index) {
                    if (s < need) {
                        lds.g.sel_key[base + gt + s] = key;
                        lds.g.sel_idx[base + gt + s] = idx;
                    }
                } else if (s < kTopkCand) {
                    tie[s] = idx;
                }
            }
        });
        __syncthreads();
        if (by_index) {
            int tp = 1;
            while (tp < last) tp <<= 1;
            for (int i = tid; i < tp; i += kTopkThreads) {
                lds.g.cand_key[i] = 0u;  // equal keys: the sort orders by index
                lds.g.cand_idx[i] = i < last ? tie[i] : 0x7fffffff;
            }
            __syncthreads();
            lds_bitonic_sort(lds.g.cand_key, lds.g.cand_idx, tp);
            for (int i = tid; i < need; i += kTopkThreads) {
                lds.g.sel_key[base + gt + i] = prefix;
                lds.g.sel_idx[base + gt + i] = lds.g.cand_idx[i];
            }
            __syncthreads();
        }
    };

    // Gather of the multi-pass path: entries above the prefix in any
    // order, tied entries in index order.
    auto gather_in_order = [&]() {
        const int greater = K - need;
        int ties_taken = 0;
        auto take_greater = [&](uint32_t key, int idx) {
            if ((key & mask) > prefix) {
                const int s = atomicAdd(&n_greater, 1);  // < greater by the select invariant
                if (s < greater) {
                    lds.g.sel_key[s] = key;
                    lds.g.sel_idx[s] = idx;
                }
            }
        };
        // One chunk of up to 4 consecutive entries per thread, chunks in index order.
        auto chunk = [&](const uint32_t (&key)[4], int idx0, int cnt) {
            int t = 0;
            for (int e = 0; e < cnt; ++e) {
                take_greater(key[e], idx0 + e);
                t += (key[e] & mask) == prefix;
            }
            if (ties_taken < need) {  // uniform
                int total;
                int rank = ties_taken + block_exclusive_sum(t, scratch, total);
                for (int e = 0; e < cnt; ++e)
                    if ((key[e] & mask) == prefix) {
                        if (rank < need) {
                            lds.g.sel_key[greater + rank] = key[e];
                            lds.g.sel_idx[greater + rank] = idx0 + e;
                        }
                        ++rank;
                    }
                ties_taken += total;
            }
        };
        {
            uint32_t k4[4] = {0u, 0u, 0u, 0u};
            if (tid < head) k4[0] = order_key(x[tid]);
            chunk(k4, tid, tid < head ? 1 : 0);
        }
        for (int i0 = 0; i0 < nvec; i0 += kTopkThreads) {
            const int j = i0 + tid;
            uint32_t k4[4] = {0u, 0u, 0u, 0u};
            int cnt = 0;
            if (j < nvec) {
                const float4 v = xv[j];
                k4[0] = order_key(v.x);
                k4[1] = order_key(v.y);
                k4[2] = order_key(v.z);
                k4[3] = order_key(v.w);
                cnt = 4;
            }
            chunk(k4, head + 4 * j, cnt);
        }
        for (int i0 = tail0; i0 < V; i0 += kTopkThreads) {
            uint32_t k4[4] = {0u, 0u, 0u, 0u};
            const int i = i0 + tid;
            if (i < V) k4[0] = order_key(x[i]);
            chunk(k4, i, i < V ? 1 : 0);
        }
        __syncthreads();
    };

    // One-read path (K <= 64, rows of 16384 entries or more). The row
    // streams in batches of 16384 entries (4 float4 per thread). Batches 0
    // to 3 go out at once; once they are in, batch 4 goes out and each
    // thread's largest entry in the full ones among them (up to 64
    // entries) gives 1024 distinct entries: the bin of their K-th largest
    // key (4096-bin histogram of the top 12 key bits, searched downward
    // from the top bin by one wave) bounds the row's K-th largest from
    // below. Then the batches are tested against the bound as they come,
    // five in flight, and the entries at or above it join one list in LDS
    // (one LDS atomic per wave and element position that has any, ballot
    // compaction inside the wave). Selection: by rank for up to 256
    // candidates; else chunks of 64 sorted in registers and a tree of
    // bitonic merges between waves, which leaves the row's 64 largest, in
    // order, in wave 0. A list that would overflow sends the row to the
    // paths below.
    if (K <= kTopkSmallK && nvec >= kTopkBatchVec) {
        const int lane = tid & 63, wave = tid >> 6;
        const int nb = (nvec + kTopkBatchVec - 1) / kTopkBatchVec;
        const int nfull = nvec / kTopkBatchVec;  // batches without re-read vectors
        // The last batch re-reads the row's last vector past its end.
        auto load = [&](int b, float4 (&d)[kTopkUnroll]) {
#pragma unroll
            for (int u = 0; u < kTopkUnroll; ++u) d[u] = xv[min(b * kTopkBatchVec + u * kTopkThreads + tid, nvec - 1)];
        };
        float4 r0[kTopkUnroll], r1[kTopkUnroll], r2[kTopkUnroll], r3[kTopkUnroll], r4[kTopkUnroll];
        load(0, r0);
        if (nb > 1) load(1, r1);
        if (nb > 2) load(2, r2);
        if (nb > 3) load(3, r3);
        for (int i = tid; i < 4096; i += kTopkThreads) hist[i] = 0u;
        if (tid == 0) {
            top_key = 0u;
            list_len = 0;
        }
        __syncthreads();
        {
            // Largest of the thread's entries in the first full batches (up
            // to four, 16 entries each, all inside the row), as a key. On
            // the raw bits as signed integers: with any entry of sign 0 the
            // largest integer is the largest value, else the smallest
            // integer is (the negative value nearest zero).
            int imax = INT_MIN, imin = INT_MAX;
            auto fold = [&](const float4 (&d)[kTopkUnroll]) {
#pragma unroll
                for (int u = 0; u < kTopkUnroll; ++u) {
                    const int a = __float_as_int(d[u].x), b = __float_as_int(d[u].y);
                    const int c = __float_as_int(d[u].z), e = __float_as_int(d[u].w);
                    imax = max(max(imax, a), b);
                    imax = max(max(imax, c), e);
                    imin = min(min(imin, a), b);
                    imin = min(min(imin, c), e);
                }
            };
            fold(r0);
            if (nfull > 1) fold(r1);
            if (nfull > 2) fold(r2);
            if (nfull > 3) fold(r3);
            const float mx = __int_as_float(imax >= 0 ? imax : imin);
            // Batches 0 to 3 have landed: batch 4 goes out now, so that it
            // streams in while the bound is found.
            __builtin_amdgcn_sched_barrier(0);
            if (nb > 4) load(4, r4);
            __builtin_amdgcn_sched_barrier(0);
            const uint32_t key = order_key(mx);
            atomicAdd(&hist[key >> 20], 1u);
            uint32_t wmax = key;
            wmax = max(wmax, lane_xor<1>(wmax));
            wmax = max(wmax, lane_xor<2>(wmax));
            wmax = max(wmax, lane_xor<4>(wmax));
            wmax = max(wmax, lane_xor<8>(wmax));
            wmax = max(wmax, lane_xor<16>(wmax));
            wmax = max(wmax, lane_xor<32>(wmax));
            if (lane == 0) atomicMax(&top_key, wmax);
        }
        __syncthreads();
        if (wave == 0) {
            // Bins from the top one down, 64 at a time (lane l: bin top - l):
            // the first bin where the count from the top reaches K. The
            // 1024 counted keys guarantee one.
            int top = (int)(top_key >> 20), above = 0, bin = 0;
            for (; top >= 0; top -= 64) {
                const int c = top - lane >= 0 ? (int)hist[top - lane] : 0;
                int s = c;
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const int y = __shfl_up(s, d, 64);
                    if (lane >= d) s += y;
                }
                const uint64_t m = __builtin_amdgcn_ballot_w64(above + s >= K);
                if (m) {
                    bin = top - __builtin_ctzll(m);
                    break;
                }
                above += __shfl(s, 63, 64);
            }
            if (lane == 0) found[0] = bin;
        }
        __syncthreads();
        // No entry has key 0x7FFFFFFF (-0.0 maps to +0.0's key): lowering a
        // bound of 0x80000000 by one admits nothing more.
        const uint32_t lo = ((uint32_t)found[0] << 20) - (found[0] == 2048 ? 1u : 0u);
        // key >= lo as one compare of the raw bits u: for a positive bound,
        // (int)u >= (int)(lo & 0x7FFFFFFF); else u <= ~lo (unsigned).
        const bool positive = lo > 0x80000000u;
        const int lo_bits = (int)(lo & 0x7FFFFFFFu);
        const uint32_t not_lo = ~lo;
        // The histogram's space now holds the ranks of the candidates.
        uint32_t *const rank = hist;
        if (tid < kTopkRankMax) rank[tid] = 0u;
        // One test per float4 (the largest, or smallest, of its four words
        // against the bound); the rare vectors that pass are split up by
        // topk_append4, which also drops the re-read copies of the row's
        // last vector (their indices lie past the body's end).
        auto process_as = [&](auto pos, int b, const float4 (&d)[kTopkUnroll]) {
            constexpr bool POS = decltype(pos)::value;
#pragma unroll
            for (int u = 0; u < kTopkUnroll; ++u) {
                const uint32_t w[4] = {__float_as_uint(d[u].x), __float_as_uint(d[u].y),
                                       __float_as_uint(d[u].z), __float_as_uint(d[u].w)};
                const bool any = POS ? max(max((int)w[0], (int)w[1]), max((int)w[2], (int)w[3])) >= lo_bits
                                     : min(min(w[0], w[1]), min(w[2], w[3])) <= not_lo;
                if (__builtin_amdgcn_ballot_w64(any))
                    topk_append4(w[0], w[1], w[2], w[3], head + 4 * (b * kTopkBatchVec + u * kTopkThreads + tid),
                                 tail0, POS, lo_bits, not_lo);
            }
        };
        auto process = [&](int b, const float4 (&d)[kTopkUnroll]) {
            if (positive)
                process_as(std::true_type{}, b, d);
            else
                process_as(std::false_type{}, b, d);
        };
        for (int b = 0; b < nb; b += 5) {
            process(b, r0);
            if (b + 5 < nb) load(b + 5, r0);
            if (b + 1 < nb) process(b + 1, r1);
            if (b + 6 < nb) load(b + 6, r1);
            if (b + 2 < nb) process(b + 2, r2);
            if (b + 7 < nb) load(b + 7, r2);
            if (b + 3 < nb) process(b + 3, r3);
            if (b + 8 < nb) load(b + 8, r3);
            if (b + 4 < nb) process(b + 4, r4);
            if (b + 9 < nb) load(b + 9, r4);
        }
        if (head > 0 || tail0 < V) {
            // The scalar head and tail: 0 .. 3 entries each, one per thread.
            const int i = tid < head ? tid : tail0 + tid - 4;
            const bool in = tid < head || (tid >= 4 && i < V);
            const uint32_t h = in ? __float_as_uint(x[i]) : 0u;
            if (__builtin_amdgcn_ballot_w64(in))
                topk_append4(h, 0u, 0u, 0u, in ? i : 0, in ? i + 1 : 0, positive, lo_bits, not_lo);
        }
        __syncthreads();
        const int total = list_len;
        if (total <= kTopkRankMax) {
            // Few candidates: each one's rank is the number of larger
            // ones (the words are distinct), counted by all 16 waves, each
            // taking one chunk of 64 candidates against one share of the
            // list; the K of rank below K go straight to their places.
            // Wave-uniform arithmetic (shifts: 1, 2 or 4 chunks, in 16, 8
            // or 4 shares).
            const int uw = __builtin_amdgcn_readfirstlane(wave);
            const int cshift = total <= 64 ? 0 : total <= 128 ? 1 : 2;
            const int chunk = uw & ((1 << cshift) - 1), part = uw >> cshift;
            {
                const int g = 64 * chunk + lane;
                const uint64_t mine = g < total ? lds.list[g] : ~0ull;
                const int share = (total + (15 >> cshift)) >> (4 - cshift);  // ceil(total / parts)
                const int j0 = min(part * share, total), j1 = min(j0 + share, total);
                uint32_t larger = 0u;
                int j = j0;
                for (; j + 8 <= j1; j += 8) {  // eight broadcast reads in flight
                    uint64_t o[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) o[u] = lds.list[j + u];
#pragma unroll
                    for (int u = 0; u < 8; ++u) larger += o[u] > mine;
                }
                for (; j < j1; ++j) larger += lds.list[j] > mine;
                if (g < total && larger) atomicAdd(&rank[g], larger);
            }
            __syncthreads();
            if (tid < total) {
                const uint32_t r = rank[tid];
                if (r < (uint32_t)K) {
                    const uint64_t wd = lds.list[tid];
                    p.values[(int64_t)blockIdx.x * K + r] = entry_value(wd);
                    p.indices[(int64_t)blockIdx.x * K + r] = entry_index(wd);
                }
            }
            return;
        }
        if (total <= kTopkListCap) {
            // The list cut into chunks of 64; wave w sorts chunks w, w + 16,
            // .. and keeps the 64 largest, descending (0 pads).
            const int nchunks = (total + 63) >> 6;
            uint32_t th = 0u, tl = 0u;
            for (int c = wave; c < nchunks; c += kTopkThreads / 64) {
                const int g = 64 * c + lane;
                const uint64_t v = g < total ? lds.list[g] : 0ull;
                uint32_t h = (uint32_t)(v >> 32), l = (uint32_t)v;
                wave_sort_desc(h, l);
                if (c == wave) {
                    th = h;
                    tl = l;
                } else {
                    wave_keep_top(th, tl, (uint32_t)__shfl((int)h, 63 - lane, 64), (uint32_t)__shfl((int)l, 63 - lane, 64));
                }
            }
            // Tree of merges over the waves that hold a list: at level s,
            // wave w + s hands its list to wave w (w a multiple of 2s)
            // through LDS (the histogram's space).
            const int nlists = min(nchunks, kTopkThreads / 64);
            uint64_t *const xbuf = reinterpret_cast<uint64_t *>(hist);
            for (int s = 1; s < nlists; s <<= 1) {
                if ((wave & (2 * s - 1)) == s && wave < nlists) xbuf[wave * 64 + lane] = ((uint64_t)th << 32) | tl;
                __syncthreads();
                if ((wave & (2 * s - 1)) == 0 && wave + s < nlists) {
                    const uint64_t o = xbuf[(wave + s) * 64 + 63 - lane];
                    wave_keep_top(th, tl, (uint32_t)(o >> 32), (uint32_t)o);
                }
            }
            if (wave == 0 && lane < K) {
                const uint64_t wd = ((uint64_t)th << 32) | tl;
                p.values[(int64_t)blockIdx.x * K + lane] = entry_value(wd);
                p.indices[(int64_t)blockIdx.x * K + lane] = entry_index(wd);
            }
            return;
        }
    }

    bool done = false;
    // Single-read path for rows longer than 16384 entries. The bin of the
    // K-th largest entry of the first chunk (8192 entries) bounds the row's
    // K-th largest from below, so one read that keeps every entry of that
    // bin or above as a candidate finds all K (on 128256-entry frequency
    // rows with K = 50: about 800 candidates). With more than kTopkCand
    // candidates (heavily tied rows, or a chunk unrepresentative of its
    // row) the two-read path below runs instead.
    const int nv0 = min(nvec, kTopkChunkVec);
    if (head + 4 * nv0 >= K && nvec > 2 * nv0) {
        for (int i = tid; i < 4096; i += kTopkThreads) hist[i] = 0u;
        __syncthreads();
        if (tid < head) atomicAdd(&hist[order_key(x[tid]) >> 20], 1u);
        for (int j = tid; j < nv0; j += kTopkThreads) {
            const float4 v = xv[j];
            atomicAdd(&hist[order_key(v.x) >> 20], 1u);
            atomicAdd(&hist[order_key(v.y) >> 20], 1u);
            atomicAdd(&hist[order_key(v.z) >> 20], 1u);
            atomicAdd(&hist[order_key(v.w) >> 20], 1u);
        }
        __syncthreads();
        find_bin(4096, K);
        const uint32_t lo = (uint32_t)found[0] << 20;
        if (tid == 0) n_cand = 0;
        __syncthreads();
        for_each([&](uint32_t key, int idx) {
            if (key >= lo) {
                const int s = atomicAdd(&n_cand, 1);
                if (s < kTopkCand) {
                    lds.g.cand_key[s] = key;
                    lds.g.cand_idx[s] = idx;
                }
            }
        });
        __syncthreads();
        const int nc = n_cand;  // >= K: the chunk alone has K entries at or above lo
        __syncthreads();        // n_cand is reset below
        if (nc <= kTopkCand) {
            pick(nc, 0, K);
            done = true;
        }
    }

    if (!done) {
        // Histogram of the top 12 bits over the whole row.
        prefix = 0u;
        mask = 0u;
        need = K;
        const int in_bin = radix_pass(0, visit_row);
        const int greater = K - need;  // how many entries lie above the prefix
        if (tid == 0) {
            n_greater = 0;
            n_cand = 0;
        }
        __syncthreads();
        if (in_bin <= kTopkCand) {
            // Second read: entries above the prefix, and the bin's entries as candidates.
            for_each([&](uint32_t key, int idx) {
                const uint32_t k = key & mask;
                if (k > prefix) {
                    const int s = atomicAdd(&n_greater, 1);  // < greater by the select invariant
                    if (s < greater) {
                        lds.g.sel_key[s] = key;
                        lds.g.sel_idx[s] = idx;
                    }
                } else if (k == prefix) {
                    const int s = atomicAdd(&n_cand, 1);  // < in_bin
                    if (s < kTopkCand) {
                        lds.g.cand_key[s] = key;
                        lds.g.cand_idx[s] = idx;
                    }
                }
            });
            __syncthreads();
            pick(in_bin, greater, need);
        } else {
            for (int pass = 1; pass < 3; ++pass)
                if (radix_pass(pass, visit_row) == need) break;  // every entry sharing the prefix is wanted
            gather_in_order();
        }
    }

    // Order the K chosen pairs, padded to a power of two with pairs that sort last.
    int kp = 1;
    while (kp < K) kp <<= 1;
    if (tid >= K && tid < kp) {
        lds.g.sel_key[tid] = 0u;
        lds.g.sel_idx[tid] = 0x7fffffff;
    }
    __syncthreads();
    lds_bitonic_sort(lds.g.sel_key, lds.g.sel_idx, kp);

    if (tid < K) {
        const int idx = lds.g.sel_idx[tid];
        p.values[(int64_t)blockIdx.x * K + tid] = x[idx];
        p.indices[(int64_t)blockIdx.x * K + tid] = idx;
    }
}

}  // namespace fa355
